// Tiled paged attention on bf16 MFMA (gfx950), producing partial softmax
// states. One kernel serves three roles:
//   * the prefix phase: every query row of the batch (all requests' tokens
//     packed as one sequence, times the query heads of one KV head) attends
//     non-causally to the shared-prefix pages (block-table row 0);
//   * the suffix phase: each request's rows attend causally to its own KV
//     range [key_start, seq_len) through its block-table row;
//   * the non-cascade path: the suffix phase with key_start = 0.
// ("vLLM Cascade Attention：用法、场景与原理解析", beaiera.top, section 8
// Step 5, phases 1 and 2; section 4 for which keys each query sees.)
//
// Work-group: 4 wave64s. A work-group owns one (KV head, row tile, KV split)
// item; its K/V range is staged through LDS 64 keys (4 pages) at a time,
// double buffered, and every wave computes 16*RB rows against each tile:
//   S^T[key][row] = K Q^T   (v_mfma_f32_16x16x32_bf16, A = K from LDS,
//                            B = Q^T held in registers)
//   online softmax on S^T (exp2 domain, fp32), P^T rounded to bf16
//   O^T[d][row] += V^T P^T (v_mfma_f32_16x16x32_bf16, A = V^T from a
//                            transposed LDS tile, B = P^T straight from the
//                            S^T accumulators)
// Computing the transposed products keeps P in the lane layout the second
// product needs, so no cross-lane shuffle of P is required. K/V positions
// outside the item's range are never read: their LDS slots are zero-filled
// and their scores masked, so NaN in unused pages or tail slots cannot leak.
#pragma once

#include "device_common.hpp"

namespace ca {

struct TileArgs {
  const uint16_t* q;            // [T][hq][D] bf16 bits
  const uint16_t* k;            // paged cache, element strides below
  const uint16_t* v;
  int64_t sp, st, sh;           // page, token-slot, head strides (elements)
  const int32_t* bt;            // [num_reqs][bt_stride]
  const int32_t* qsl;           // [num_reqs + 1]
  const int32_t* seq_lens;      // [num_reqs]
  int32_t bt_stride;
  int32_t hq, hkv, group;
  float scale_log2;             // softmax_scale * log2(e)
  int32_t prefix_mode;          // 1: prefix phase, 0: per-request phase
  int32_t total_rows;           // prefix: T * group
  int32_t key_start;            // per-request phase: first KV position
  int32_t prefix_len;           // prefix phase: number of shared KV positions
  int32_t num_reqs;
  int32_t mtiles;               // row tiles (prefix) / max row tiles per request
  int32_t splits;               // KV splits (prefix) / chunks per request
  int32_t split_tokens;         // multiple of 64
  float* part_o;                // [slots][T][hq][D] fp32 (partial mode)
  float* part_lse;              // [slots][T][hq] fp32, natural log
  int32_t slot_base;
  int64_t slot_elems;           // T * hq * D
  int64_t slot_rows;            // T * hq
  uint16_t* out;                // [T][hq][D] bf16 (direct mode)
  float* lse_out;               // [T][hq] (direct mode, may be null)
  int32_t direct;
};

template <int D>
struct TileSmem {
  static constexpr int KS = D + 8;        // K row stride (elements): 16-byte rows, spread banks
  static constexpr int VS = 64 + 8;       // V^T row stride (elements)
  static constexpr int K_ELEMS = 64 * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int BUF = K_ELEMS + V_ELEMS;
  static constexpr int BYTES = 2 * BUF * 2;
};

template <int D, int RB>
__global__ __launch_bounds__(256) void attn_tile_kernel(const TileArgs a) {
  constexpr int KC = D / 32;              // 32-wide d chunks per QK^T MFMA chain
  constexpr int DB = D / 16;              // 16-wide d blocks of the output
  constexpr int KCH = D / 8;              // 16-byte chunks per K/V row
  constexpr int K_LOADS = 64 * KCH / 256; // per thread per tile
  constexpr int V_ITEMS = 16 * KCH;       // (key quad, d chunk) pairs per tile
  constexpr int V_LOADS = (V_ITEMS + 255) / 256;
  using SM = TileSmem<D>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * SM::BUF];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int lr = lane & 15;
  const int lq = lane >> 4;

  // ---------------------------------------------------------- item decode
  int g, row_begin, row_end, key_begin, key_end, slot, req = 0;
  int tok_base = 0, q_pos_base = 0;      // token of row 0, causal position of row 0's token
  bool causal;
  const int32_t* bt_row;
  {
    const int bid = blockIdx.x;
    if (a.prefix_mode) {
      const int kv_items = a.hkv * a.splits;
      const int mt = bid / kv_items;
      const int kvi = bid - mt * kv_items;
      g = kvi / a.splits;
      const int s = kvi - g * a.splits;
      row_begin = mt * 64 * RB;
      row_end = min(row_begin + 64 * RB, a.total_rows);
      key_begin = s * a.split_tokens;
      key_end = min(key_begin + a.split_tokens, a.prefix_len);
      slot = a.slot_base + s;
      causal = false;
      bt_row = a.bt;
    } else {
      const int c = bid % a.splits;
      int rest = bid / a.splits;
      const int mt = rest % a.mtiles;
      rest /= a.mtiles;
      g = rest % a.hkv;
      req = rest / a.hkv;
      const int q0 = a.qsl[req];
      const int q_len = a.qsl[req + 1] - q0;
      const int seq_len = a.seq_lens[req];
      row_begin = mt * 64 * RB;
      row_end = min(row_begin + 64 * RB, q_len * a.group);
      if (row_begin >= row_end) return;   // uniform across the work-group
      key_begin = a.key_start + c * a.split_tokens;
      key_end = min(key_begin + a.split_tokens, seq_len);
      if (key_end < key_begin) key_end = key_begin;
      slot = a.slot_base + c;
      causal = true;
      tok_base = q0;
      q_pos_base = seq_len - q_len;          // num_computed_tokens
      bt_row = a.bt + (int64_t)req * a.bt_stride;
    }
  }
  const int n_tiles = (key_end - key_begin + 63) >> 6;

  // ------------------------------------------------- per-lane query rows
  const int wrow0 = row_begin + wave * 16 * RB;
  const bool wave_active = wrow0 < row_end;
  u32x4_t qf[RB][KC];
  int row_tok[RB], row_head[RB], row_qpos[RB];
  bool row_ok[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const int m = wrow0 + rb * 16 + lr;
    row_ok[rb] = m < row_end;
    const int mt = a.prefix_mode ? m : m;            // packed row index within the item space
    const int t_in = mt / a.group;
    const int j = mt - t_in * a.group;
    row_tok[rb] = tok_base + t_in;
    row_head[rb] = g * a.group + j;
    row_qpos[rb] = q_pos_base + t_in;
#pragma unroll
    for (int kc = 0; kc < KC; ++kc) {
      if (row_ok[rb]) {
        qf[rb][kc] = load16(a.q + ((int64_t)row_tok[rb] * a.hq + row_head[rb]) * D + kc * 32 + lq * 8);
      } else {
        qf[rb][kc] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
  }

  f32x4_t o[DB][RB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) o[db][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  float m_run[RB], l_run[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m_run[rb] = -INFINITY;
    l_run[rb] = 0.f;
  }

  // ------------------------------------------------ global -> register stage
  u32x4_t kreg[K_LOADS];
  u32x4_t vreg[V_LOADS][4];
  const int64_t head_off = (int64_t)g * a.sh;

  auto load_tile = [&](int t) {
    const int kt0 = key_begin + t * 64;
    int pg[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) pg[kb] = (kt0 + kb * 16 < key_end) ? bt_row[(kt0 >> 4) + kb] : 0;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = tid + 256 * i;
      const int key = c / KCH;
      const int dc = c - key * KCH;
      const int pos = kt0 + key;
      if (pos < key_end) {
        kreg[i] = load16(a.k + (int64_t)pg[key >> 4] * a.sp + (int64_t)(pos & 15) * a.st + head_off + dc * 8);
      } else {
        kreg[i] = u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int c = tid + 256 * i;
      const int kq = c / KCH;
      const int dc = c - kq * KCH;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const int key = kq * 4 + kk;
        const int pos = kt0 + key;
        if (c < V_ITEMS && pos < key_end) {
          vreg[i][kk] = load16(a.v + (int64_t)pg[key >> 4] * a.sp + (int64_t)(pos & 15) * a.st + head_off + dc * 8);
        } else {
          vreg[i][kk] = u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* sK = smem + buf * SM::BUF;
    uint16_t* sV = sK + SM::K_ELEMS;
#pragma unroll
    for (int i = 0; i < K_LOADS; ++i) {
      const int c = tid + 256 * i;
      const int key = c / KCH;
      const int dc = c - key * KCH;
      *reinterpret_cast<u32x4_t*>(sK + key * SM::KS + dc * 8) = kreg[i];
    }
#pragma unroll
    for (int i = 0; i < V_LOADS; ++i) {
      const int c = tid + 256 * i;
      if (c < V_ITEMS) {
        const int kq = c / KCH;
        const int dc = c - kq * KCH;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          const int sh = (e & 1) * 16;
          const uint32_t x0 = (vreg[i][0][w] >> sh) & 0xffffu;
          const uint32_t x1 = (vreg[i][1][w] >> sh) & 0xffffu;
          const uint32_t x2 = (vreg[i][2][w] >> sh) & 0xffffu;
          const uint32_t x3 = (vreg[i][3][w] >> sh) & 0xffffu;
          *reinterpret_cast<u32x2_t*>(sV + (dc * 8 + e) * SM::VS + kq * 4) = u32x2_t{x0 | (x1 << 16), x2 | (x3 << 16)};
        }
      }
    }
  };

  if (n_tiles > 0) load_tile(0);
  for (int t = 0; t < n_tiles; ++t) {
    const int buf = t & 1;
    store_tile(buf);
    __syncthreads();
    if (t + 1 < n_tiles) load_tile(t + 1);
    if (wave_active) {
      const uint16_t* sK = smem + buf * SM::BUF;
      const uint16_t* sV = sK + SM::K_ELEMS;
      const int kt0 = key_begin + t * 64;
      // S^T = K Q^T for 4 blocks of 16 keys
      f32x4_t s[4][RB];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[kb][rb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kc = 0; kc < KC; ++kc) {
          const u32x4_t kf = *reinterpret_cast<const u32x4_t*>(sK + (kb * 16 + lr) * SM::KS + kc * 32 + lq * 8);
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) s[kb][rb] = mfma16x16x32(kf, qf[rb][kc], s[kb][rb]);
        }
      }
      // online softmax over this tile's 64 keys, per row (lane lr)
      u32x4_t pb[RB][2];
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        float x[4][4];
        float tmax = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int kpos = kt0 + kb * 16 + lq * 4 + i;
            const bool vis = kpos < key_end && (!causal || kpos <= row_qpos[rb]);
            x[kb][i] = vis ? s[kb][rb][i] * a.scale_log2 : -INFINITY;
            tmax = fmaxf(tmax, x[kb][i]);
          }
        tmax = wave_max_across_quads(tmax);
        const float m_new = fmaxf(m_run[rb], tmax);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = exp2f(m_run[rb] - m_use);
        float psum = 0.f;
        float p[4][4];
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            p[kb][i] = exp2f(x[kb][i] - m_use);
            psum += p[kb][i];
          }
        l_run[rb] = l_run[rb] * alpha + psum;
        m_run[rb] = m_new;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db][rb] *= alpha;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          pb[rb][kk] = u32x4_t{pack_bf16x2(p[2 * kk][0], p[2 * kk][1]), pack_bf16x2(p[2 * kk][2], p[2 * kk][3]),
                               pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]),
                               pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3])};
        }
      }
      // O^T += V^T P^T, 32 keys per MFMA: k-slot (lq, j) <-> key
      // kk*32 + (j < 4 ? 4*lq + j : 16 + 4*lq + j - 4), the same map the
      // S^T accumulators give P^T.
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
          const uint16_t* vrow = sV + (db * 16 + lr) * SM::VS + kk * 32 + lq * 4;
          const u32x2_t lo = *reinterpret_cast<const u32x2_t*>(vrow);
          const u32x2_t hi = *reinterpret_cast<const u32x2_t*>(vrow + 16);
          const u32x4_t vf = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
#pragma unroll
          for (int rb = 0; rb < RB; ++rb) o[db][rb] = mfma16x16x32(vf, pb[rb][kk], o[db][rb]);
        }
      }
    }
  }

  // ------------------------------------------------------------ epilogue
  if (!wave_active) return;
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const float l_tot = wave_sum_across_quads(l_run[rb]);
    const bool live = l_tot > 0.f;
    const float inv = live ? 1.f / l_tot : 0.f;
    const float lse = live ? (m_run[rb] + log2f(l_tot)) * kLn2 : -INFINITY;
    if (!row_ok[rb]) continue;
    const int64_t row = (int64_t)row_tok[rb] * a.hq + row_head[rb];
    if (a.direct) {
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const f32x4_t v = o[db][rb] * inv;
        *reinterpret_cast<u32x2_t*>(a.out + row * D + db * 16 + lq * 4) =
            u32x2_t{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
      }
      if (lq == 0 && a.lse_out) a.lse_out[row] = lse;
    } else {
      float* dst = a.part_o + (int64_t)slot * a.slot_elems + row * D;
#pragma unroll
      for (int db = 0; db < DB; ++db) *reinterpret_cast<f32x4_t*>(dst + db * 16 + lq * 4) = o[db][rb] * inv;
      if (lq == 0) a.part_lse[(int64_t)slot * a.slot_rows + row] = lse;
    }
  }
}

}  // namespace ca
