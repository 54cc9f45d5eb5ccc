// HIP kernels (gfx950 / MI355X) for the backward pass of prefix-masked
// attention, bf16 inputs, fp32 accumulation.
//
// The gradients are those of the forward in attn_kernels.hpp with the keys cut
// to the valid prefix j < n_b (the truncation identity of tabfm PR #80,
// section Fix, carried to the derivative); padded key slots get dk = dv = 0.
// With P = softmax(scale q k^T) recomputed from the saved natural-log LSE:
//     delta_i = sum_d dout_id out_id          (bwd_delta_kernel)
//     dS = P * (dout v^T - delta)
//     dq = scale dS k                         (bwd_dq_kernel: one workgroup per
//                                              128 query rows, walks the keys)
//     dk = scale dS^T q,  dv = P^T dout       (bwd_dkdv_kernel: one workgroup per
//                                              128 keys, walks the queries)
// No atomics: every gradient element is written once, so results are
// deterministic.  Both walking kernels reuse the forward's 64-row LDS tile
// layout, which serves plain row-fragment reads (A = rows x d) and transposed
// reads (A = d x rows) of the same tile without bank conflicts:
//   dq   : S^T = K Q^T, dP^T = V dO^T  (row reads of the K and V tiles),
//          dQ^T += K^T dS^T            (transposed reads of the K tile);
//   dkdv : S = Q K^T, dP = dO V^T      (row reads of the Q and dO tiles),
//          dV^T += dO^T P, dK^T += Q^T dS (transposed reads of the same tiles).
// In dq a lane owns one query row (as in the forward); in dkdv a lane owns one
// key row and the contraction runs over queries.
#pragma once

#include "attn_kernels.hpp"

namespace lcp {

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* kv_len;
  const void* out;
  const void* dout;
  const float* lse;  // natural-log LSE of the forward, [B,H,Tq]
  float* delta;      // [B,H,Tq], written by bwd_delta_kernel
  int B, H, Tq, S;
  float scale;
  float scale_log2;  // scale * log2(e)
  int n_tiles;       // grid decode: query tiles (dq) or key blocks (dkdv) per (b, h)
  void* dq;
  void* dk;
  void* dv;
};

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// delta[row] = sum_d dout[row][d] * out[row][d] in fp32; D/8 lanes per row, 16 bytes each.
template <int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(BwdArgs a, int64_t rows) {
  constexpr int TPR = D / 8;
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int c = threadIdx.x % TPR;
  float acc = 0.0f;
  if (row < rows) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.out) + row * D + 8 * c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint16_t*>(a.dout) + row * D + 8 * c);
#pragma unroll
    for (int i = 0; i < 4; ++i) acc += bf16_lo(o[i]) * bf16_lo(g[i]) + bf16_hi(o[i]) * bf16_hi(g[i]);
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < rows && c == 0) a.delta[row] = acc;
}

// Store 32 rows x D of fp32 accumulators (transposed MFMA layout: lane = row % 32,
// o[db][4 rg + i] = column 32 db + 8 rg + 4 h + i) times `mul` as bf16.
template <int D>
__device__ __forceinline__ void store_rows_bf16(void* base, int64_t row, const f32x16 (&o)[D / 32], float mul,
                                                int h_half) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int64_t off = row * D + 32 * db + 8 * rg + 4 * h_half;
      const u32x2 w = {pack_bf16x2(o[db][4 * rg] * mul, o[db][4 * rg + 1] * mul),
                       pack_bf16x2(o[db][4 * rg + 2] * mul, o[db][4 * rg + 3] * mul)};
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + off) = w;
    }
}

template <int D>
__device__ __forceinline__ void store_zero_rows_bf16(void* base, int64_t row, int h_half) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int64_t off = row * D + 32 * db + 8 * rg + 4 * h_half;
      *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(base) + off) = u32x2{0u, 0u};
    }
}

// ------------------------------------------------------------------ dq
// Workgroup = (128-query tile, h, b); 4 waves x 32 query rows.  Walks the valid
// key tiles with K and V double-buffered in LDS (the next pair is loaded while
// the current one is used).
template <int D, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(WPE, WPE)))
void bwd_dq_kernel(BwdArgs a) {
  using P = Bf16Dma<D>;
  __shared__ __attribute__((aligned(16))) char smem_raw[P::LDS_BYTES];
  lds_char* const smem = (lds_char*)smem_raw;
  auto kb_ = [&](int i) { return smem + i * P::TILE_BYTES; };        // K buffers 0, 1
  auto vb_ = [&](int i) { return smem + (2 + i) * P::TILE_BYTES; };  // V buffers 0, 1

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h_half = lane >> 5;
  int wg = blockIdx.x;
  const int qt = wg % a.n_tiles;
  wg /= a.n_tiles;
  const int h = wg % a.H, b = wg / a.H;
  int n = a.kv_len[b];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  const int64_t bh = (int64_t)b * a.H + h;
  const int row = qt * kBM + wave * 32 + (lane & 31);
  const bool row_ok = row < a.Tq;
  const int64_t grow = bh * a.Tq + row;
  if (n == 0) {  // no valid key: the output is the constant 0
    if (row_ok) store_zero_rows_bf16<D>(a.dq, grow, h_half);
    return;
  }
  const int T = (n + kBN - 1) / kBN;
  auto nv_of = [&](int t) {
    const int r = n - t * kBN;
    return r < 0 ? 0 : (r > kBN ? kBN : r);
  };
  const uint16_t* kg = reinterpret_cast<const uint16_t*>(a.k) + bh * a.S * D;
  const uint16_t* vg = reinterpret_cast<const uint16_t*>(a.v) + bh * a.S * D;
  auto k_tile = [&](int t) { return make_rsrc(kg + (int64_t)t * kBN * D, (uint32_t)nv_of(t) * (D * 2)); };
  auto v_tile = [&](int t) { return make_rsrc(vg + (int64_t)t * kBN * D, (uint32_t)nv_of(t) * (D * 2)); };

  typename P::QFrag qf, gf;
  const int64_t src_row = bh * a.Tq + (row_ok ? row : 0);
  P::load_q(qf, reinterpret_cast<const uint16_t*>(a.q) + src_row * D, row_ok, h_half);
  P::load_q(gf, reinterpret_cast<const uint16_t*>(a.dout) + src_row * D, row_ok, h_half);
  const float L = row_ok ? a.lse[grow] * kLog2e : 0.0f;  // rows past Tq compute finite junk, never stored
  const float dl = row_ok ? a.delta[grow] : 0.0f;
  const float c = a.scale_log2;
  const int kbase = P::k_base(lane);
  const int vbase = P::v_base(lane);

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  P::dma_tile(k_tile(0), kb_(0), wave_u, lane);
  P::dma_tile(v_tile(0), vb_(0), wave_u, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    if (t + 1 < T) {  // the other buffers were last read before the previous barrier
      P::dma_tile(k_tile(t + 1), kb_(cur ^ 1), wave_u, lane);
      P::dma_tile(v_tile(t + 1), vb_(cur ^ 1), wave_u, lane);
    }
    f32x16 s[kBN / 32], dp[kBN / 32];
    P::scores(s, qf, kb_(cur), kbase);   // S^T = K Q^T
    P::scores(dp, gf, vb_(cur), kbase);  // dP^T = V dO^T
    const int nv = nv_of(t);
    u32x4 pk[kBN / 16];
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks) {
      float d8[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int kb = ks >> 1, r = 8 * (ks & 1) + e;
        float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -L));
        if (st_key(kb, r, h_half) >= nv) p = 0.0f;  // keys past n_b in the last tile
        d8[e] = p * (dp[kb][r] - dl);
      }
      pk[ks] = u32x4{pack_bf16x2(d8[0], d8[1]), pack_bf16x2(d8[2], d8[3]), pack_bf16x2(d8[4], d8[5]),
                     pack_bf16x2(d8[6], d8[7])};
    }
    P::accumulate(acc, pk, kb_(cur), vbase);  // dQ^T += K^T dS^T
    __builtin_amdgcn_s_waitcnt(0x0F70);       // the next tiles have landed in LDS
    lds_barrier();
  }
  if (row_ok) store_rows_bf16<D>(a.dq, grow, acc, a.scale, h_half);
}

// ---------------------------------------------------------------- dk, dv
// Workgroup = (128-key block, h, b); 4 waves x 32 keys, each lane owning one key
// row whose k and v stay in registers.  Walks every query tile (64 rows) with Q,
// dO and the tile's LSE / delta double-buffered in LDS.  Key rows at or past n_b
// are written as zeros.
template <int D, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(WPE, WPE)))
void bwd_dkdv_kernel(BwdArgs a) {
  using P = Bf16Dma<D>;
  constexpr int kKeysPerWg = 128;
  __shared__ __attribute__((aligned(16))) char smem_raw[P::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float stat[2][2][kBN];  // [buffer][lse*log2e | delta][query]
  lds_char* const smem = (lds_char*)smem_raw;
  auto qb_ = [&](int i) { return smem + i * P::TILE_BYTES; };        // Q buffers 0, 1
  auto gb_ = [&](int i) { return smem + (2 + i) * P::TILE_BYTES; };  // dO buffers 0, 1

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h_half = lane >> 5;
  int wg = blockIdx.x;
  const int kblk = wg % a.n_tiles;
  wg /= a.n_tiles;
  const int h = wg % a.H, b = wg / a.H;
  int n = a.kv_len[b];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  const int64_t bh = (int64_t)b * a.H + h;
  const int key = kblk * kKeysPerWg + wave * 32 + (lane & 31);
  const bool key_in = key < a.S;  // an allocated slot (its gradient row is written)
  const bool key_ok = key < n;    // a valid key
  const int64_t krow = bh * a.S + key;
  if (kblk * kKeysPerWg >= n || a.Tq == 0) {  // no valid key here, or no query: zero gradients
    if (key_in) {
      store_zero_rows_bf16<D>(a.dk, krow, h_half);
      store_zero_rows_bf16<D>(a.dv, krow, h_half);
    }
    return;
  }
  const int TQ = (a.Tq + kBN - 1) / kBN;
  auto nq_of = [&](int t) {
    const int r = a.Tq - t * kBN;
    return r < 0 ? 0 : (r > kBN ? kBN : r);
  };
  const uint16_t* qg = reinterpret_cast<const uint16_t*>(a.q) + bh * a.Tq * D;
  const uint16_t* gg = reinterpret_cast<const uint16_t*>(a.dout) + bh * a.Tq * D;
  auto q_tile = [&](int t) { return make_rsrc(qg + (int64_t)t * kBN * D, (uint32_t)nq_of(t) * (D * 2)); };
  auto g_tile = [&](int t) { return make_rsrc(gg + (int64_t)t * kBN * D, (uint32_t)nq_of(t) * (D * 2)); };
  const float* lse_bh = a.lse + bh * a.Tq;
  const float* del_bh = a.delta + bh * a.Tq;
  // threads 0..63 stage lse * log2e, threads 64..127 delta, for one query tile; queries
  // past Tq get lse = +inf (so P = 0) and delta = 0
  auto stat_load = [&](int t) -> float {
    const int qi = t * kBN + (tid & 63);
    if (tid < 64) return qi < a.Tq ? lse_bh[qi] * kLog2e : __builtin_inff();
    if (tid < 128) return qi < a.Tq ? del_bh[qi] : 0.0f;
    return 0.0f;
  };

  typename P::QFrag kf, vf;
  const int64_t src = bh * a.S + (key_ok ? key : 0);
  P::load_q(kf, reinterpret_cast<const uint16_t*>(a.k) + src * D, key_ok, h_half);
  P::load_q(vf, reinterpret_cast<const uint16_t*>(a.v) + src * D, key_ok, h_half);
  const float c = a.scale_log2;
  const int kbase = P::k_base(lane);
  const int vbase = P::v_base(lane);

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk[db] = f32x16{};
    dv[db] = f32x16{};
  }

  P::dma_tile(q_tile(0), qb_(0), wave_u, lane);
  P::dma_tile(g_tile(0), gb_(0), wave_u, lane);
  {
    const float x = stat_load(0);
    if (tid < 128) stat[0][tid >> 6][tid & 63] = x;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  for (int t = 0; t < TQ; ++t) {
    const int cur = t & 1;
    float next_stat = 0.0f;
    if (t + 1 < TQ) {
      P::dma_tile(q_tile(t + 1), qb_(cur ^ 1), wave_u, lane);
      P::dma_tile(g_tile(t + 1), gb_(cur ^ 1), wave_u, lane);
      next_stat = stat_load(t + 1);
    }
    f32x16 s[kBN / 32], dp[kBN / 32];
    P::scores_vgpr(s, kf, qb_(cur), kbase);   // S = Q K^T   (rows: queries of the tile, lane: key)
    P::scores_vgpr(dp, vf, gb_(cur), kbase);  // dP = dO V^T
    xdl_result_guard();
    u32x4 ppk[kBN / 16], dpk[kBN / 16];
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks) {
      const int kb = ks >> 1;
      float p8[8], d8[8];
#pragma unroll
      for (int g4 = 0; g4 < 2; ++g4) {
        // registers 8 (ks & 1) + 4 g4 + i hold queries 32 kb + 8 (2 (ks & 1) + g4) + 4 h + i
        const int q0 = 32 * kb + 8 * (2 * (ks & 1) + g4) + 4 * h_half;
        const f32x4 Lq = *reinterpret_cast<const f32x4*>(&stat[cur][0][q0]);
        const f32x4 Dq = *reinterpret_cast<const f32x4*>(&stat[cur][1][q0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = 8 * (ks & 1) + 4 * g4 + i;
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[kb][r], c, -Lq[i]));
          p8[4 * g4 + i] = p;
          d8[4 * g4 + i] = p * (dp[kb][r] - Dq[i]);
        }
      }
      ppk[ks] = u32x4{pack_bf16x2(p8[0], p8[1]), pack_bf16x2(p8[2], p8[3]), pack_bf16x2(p8[4], p8[5]),
                      pack_bf16x2(p8[6], p8[7])};
      dpk[ks] = u32x4{pack_bf16x2(d8[0], d8[1]), pack_bf16x2(d8[2], d8[3]), pack_bf16x2(d8[4], d8[5]),
                      pack_bf16x2(d8[6], d8[7])};
    }
    P::accumulate(dv, ppk, gb_(cur), vbase);  // dV^T += dO^T P
    P::accumulate(dk, dpk, qb_(cur), vbase);  // dK^T += Q^T dS
    if (t + 1 < TQ && tid < 128) stat[cur ^ 1][tid >> 6][tid & 63] = next_stat;
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the next tiles have landed in LDS
    lds_barrier();
  }
  if (key_in) {
    if (key_ok) {
      store_rows_bf16<D>(a.dk, krow, dk, a.scale, h_half);
      store_rows_bf16<D>(a.dv, krow, dv, 1.0f, h_half);
    } else {
      store_zero_rows_bf16<D>(a.dk, krow, h_half);
      store_zero_rows_bf16<D>(a.dv, krow, h_half);
    }
  }
}

}  // namespace lcp
