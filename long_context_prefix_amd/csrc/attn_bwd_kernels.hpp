// HIP kernels (gfx950 / MI355X) for the backward pass of prefix-masked
// attention, bf16 inputs, fp32 accumulation.
//
// The gradients are those of the forward in attn_kernels.hpp with the keys cut
// to the valid prefix j < n_b (the truncation identity of tabfm PR #80,
// section Fix, carried to the derivative); padded key slots get dk = dv = 0.
// With P = softmax(scale q k^T) recomputed from the saved natural-log LSE:
//     delta_i = sum_d dout_id out_id          (bwd_delta_kernel)
//     dS = P * (dout v^T - delta)
//     dq = scale dS k                         (bwd_dq_slot_kernel: one workgroup per
//                                              128 query rows, walks the keys)
//     dk = scale dS^T q,  dv = P^T dout       (bwd_dkdv_*_kernel: one workgroup per
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
  int order_b;       // 1: batch elements are walked longest prefix first (1 < B <= 64)
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
// Workgroup = (128-query tile, h, b); 4 waves x 32 query rows, walking the valid
// key tiles with K and V double-buffered in LDS (the next pair is loaded while
// the current one is used).  Each key tile is split into its two 32-key halves so
// that the softmax of one half runs on the VALU while the MFMA pipe works on the
// other: phase A issues S^T and dP^T of keys 0..31; phase B those of keys
// 32..63 while P and dS of keys 0..31 are formed; phase C accumulates
// dQ^T += K^T dS^T over keys 0..31 while P and dS of keys 32..63 are formed;
// phase D accumulates over keys 32..63.  Fixed slots separated by scheduling
// fences, with the next tiles' DMA spread over the first slots.
template <int D, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(WPE, WPE)))
void bwd_dq_slot_kernel(BwdArgs a) {
  using P = Bf16Dma<D>;
  constexpr int R = 2;                 // operand reads issued this many slots ahead
  constexpr int NH = 2 * P::NQ;        // S^T and dP^T MFMAs of one 32-key half
  constexpr int NC = (D / 32) * 2;     // dQ^T MFMAs of one 32-key half (two 16-key steps)
  constexpr int EB = (16 + NH - 1) / NH;  // softmax elements per phase B slot (16 per half)
  constexpr int EC = (16 + NC - 1) / NC;  // per phase C slot
  __shared__ __attribute__((aligned(16))) char smem_raw[P::LDS_BYTES];
  lds_char* const smem = (lds_char*)smem_raw;
  auto kb_ = [&](int i) { return smem + i * P::TILE_BYTES; };
  auto vb_ = [&](int i) { return smem + (2 + i) * P::TILE_BYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h_half = lane >> 5;
  int wg = blockIdx.x;
  const int qt = wg % a.n_tiles;
  wg /= a.n_tiles;
  const int h = wg % a.H, b = a.order_b ? longest_first(a.kv_len, a.B, a.S, wg / a.H) : wg / a.H;
  int n = a.kv_len[b];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  const int64_t bh = (int64_t)b * a.H + h;
  const int row = qt * kBM + wave * 32 + (lane & 31);
  const bool row_ok = row < a.Tq;
  const int64_t grow = bh * a.Tq + row;
  if (n == 0) {
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
  const float L = row_ok ? a.lse[grow] * kLog2e : 0.0f;
  // dP^T - delta is formed by the MFMAs: each dP^T chain starts from a block of -delta (all
  // 16 registers of a lane belong to its query row), which spares a subtraction per element
  f32x16 neg_dl;
  {
    const float dl = row_ok ? a.delta[grow] : 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) neg_dl[e] = -dl;
    asm volatile("" : "+v"(neg_dl));  // one live block, not rebuilt before every chain
  }
  float c = a.scale_log2;
  if (c < 0.0f) {  // c * (q.k) == |c| * ((-q).k): keep c > 0 so that a -inf score gives p = 0
    c = -c;
#pragma unroll
    for (int kk = 0; kk < P::NQ; ++kk) {
      u32x4 x = __builtin_bit_cast(u32x4, qf.v[kk]) ^ 0x80008000u;
      qf.v[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }
  c = fmaxf(c, 1.17549435e-38f);  // a zero scale as the smallest normal float (p = 2^-L as for scale 0)
  const int kbase = P::k_base(lane);
  const int vbase = P::v_base(lane);
  // keys at or past nv of the last tile get s = -inf, so p = 0 and dS = 0 (rare: the key
  // indices come from an opaque copy of the lane's half, so that they are computed here
  // instead of being hoisted out of the tile loop into live registers)
  auto mask_half = [&](f32x16& sh, int hf, int nv) {
    int hh = h_half;
    asm volatile("" : "+v"(hh));
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if (st_key(hf, e, hh) >= nv) sh[e] = -__builtin_inff();
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  P::dma_tile(k_tile(0), kb_(0), wave_u, lane);
  P::dma_tile(v_tile(0), vb_(0), wave_u, lane);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int t = 0; t < T; ++t) {
    const int cur = t & 1;
    const lds_char* kt = kb_(cur);
    const lds_char* vt = vb_(cur);
    // past the last tile the resources are empty: the loads zero-fill a buffer never read
    const __amdgpu_buffer_rsrc_t k_rs = k_tile(t + 1), v_rs = v_tile(t + 1);
    const int nv = nv_of(t);
    f32x16 s[2], dp[2];
    u32x4 pk[4];
    float d8[8];
    // slot j of phases A and B: MFMA j of half `hf`: j even -> S^T (A = K rows), odd ->
    // dP^T - delta (A = V rows)
    auto frag_ab = [&](int hf, int j) {
      const int kk = j >> 1;
      return P::k_frag((j & 1) ? vt : kt, kbase, 2 * kk + hf);
    };
    auto mfma_ab = [&](int hf, int j, bf16x8 fr) {
      const int kk = j >> 1;
      f32x16& d = (j & 1) ? dp[hf] : s[hf];
      if (kk == 0) {
        if (j & 1) mfma_vgpr_from(d, fr, gf.v[0], neg_dl);
        else mfma_vgpr_first(d, fr, qf.v[0]);
      } else {
        mfma_vgpr_acc(d, fr, (j & 1) ? gf.v[kk] : qf.v[kk]);
      }
    };
    // softmax element e (0..15) of half hf: register e of S^T block hf
    auto elem = [&](int hf, int e) {
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hf][e], c, -L));
      d8[e & 7] = p * dp[hf][e];
      if ((e & 7) == 7)
        pk[2 * hf + (e >> 3)] = u32x4{pack_bf16x2(d8[0], d8[1]), pack_bf16x2(d8[2], d8[3]),
                                      pack_bf16x2(d8[4], d8[5]), pack_bf16x2(d8[6], d8[7])};
    };
    // slot j of phases C and D: dQ^T block db = j % (D/32), 16-key step ks = 2 hf + j / (D/32)
    auto frag_cd = [&](int hf, int j) { return P::v_frag(kt, vbase, (2 * hf + j / (D / 32)) * (D / 32) + j % (D / 32)); };
    auto mfma_cd = [&](int hf, int j, bf16x8 fr) {
      const int db = j % (D / 32), ks = 2 * hf + j / (D / 32);
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr, __builtin_bit_cast(bf16x8, pk[ks]), acc[db], 0, 0, 0);
    };

    bf16x8 fr[R];
    // phase A: S^T, dP^T of keys 0..31, with the next tiles' DMA
#pragma unroll
    for (int i = 0; i < R; ++i) fr[i] = frag_ab(0, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      mfma_ab(0, j, fr[j % R]);
      if (j + R < NH) fr[j % R] = frag_ab(0, j + R);
      else fr[j % R] = frag_ab(1, j + R - NH);
      if (j < 2 * P::DMA_PER_WAVE) {
        if (j < P::DMA_PER_WAVE) P::dma_block(k_rs, kb_(cur ^ 1), wave_u, lane, j);
        else P::dma_block(v_rs, vb_(cur ^ 1), wave_u, lane, j - P::DMA_PER_WAVE);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    xdl_result_guard<1>();  // the softmax below reads the half-0 results
    if (nv < kBN) {
      rare_path();
      mask_half(s[0], 0, nv);
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase B: S^T, dP^T of keys 32..63; P and dS of keys 0..31
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      mfma_ab(1, j, fr[j % R]);
      if (j + R < NH) fr[j % R] = frag_ab(1, j + R);
      else fr[j % R] = frag_cd(0, j + R - NH);
#pragma unroll
      for (int u = 0; u < EB; ++u)
        if (j * EB + u < 16) elem(0, j * EB + u);
      __builtin_amdgcn_sched_barrier(0);
    }
    xdl_result_guard<1>();  // the softmax below reads the half-1 results
    if (nv < kBN) {
      rare_path();
      mask_half(s[1], 1, nv);
    }
    __builtin_amdgcn_sched_barrier(0);
    // phase C: dQ^T over keys 0..31; P and dS of keys 32..63
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      mfma_cd(0, j, fr[j % R]);
      if (j + R < NC) fr[j % R] = frag_cd(0, j + R);
      else fr[j % R] = frag_cd(1, j + R - NC);
#pragma unroll
      for (int u = 0; u < EC; ++u)
        if (j * EC + u < 16) elem(1, j * EC + u);
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase D: dQ^T over keys 32..63
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      mfma_cd(1, j, fr[j % R]);
      if (j + R < NC) fr[j % R] = frag_cd(1, j + R);
      __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // the next tiles have landed in LDS
    lds_barrier();
  }
  if (row_ok) store_rows_bf16<D>(a.dq, grow, acc, a.scale, h_half);
}

// ---------------------------------------------------------------- dk, dv
// Workgroup = (128-key block, h, b); 4 waves x 32 keys, each lane owning one key
// row whose k and v stay in registers.  Walks every query tile (64 rows) with Q,
// dO and the tile's LSE / delta double-buffered in LDS.  Key rows at or past n_b
// are written as zeros.  Each query tile is split into its two 32-query halves,
// laid out in fixed slots: phase A issues S and dP of
// queries 0..31 (and the next tiles' DMA); phase B those of queries 32..63
// while P and dS of queries 0..31 are formed; phase C accumulates dV and dK
// over queries 0..31 while P and dS of queries 32..63 are formed; phase D
// accumulates over queries 32..63.  Nothing beyond one tile's scores is held,
// so this fits D = 256 at one wave per SIMD (D = 128 uses the cross-tile
// pipelined kernel below, 2% faster there).
template <int D, int WPE>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(WPE, WPE)))
void bwd_dkdv_slot_kernel(BwdArgs a) {
  using P = Bf16Dma<D>;
  constexpr int kKeysPerWg = 128;
  constexpr int R = 2;
  constexpr int NH = 2 * P::NQ;           // S and dP MFMAs of one 32-query half
  constexpr int NC = 2 * (D / 32) * 2;    // dV and dK MFMAs of one half (two 16-query steps each)
  constexpr int EB = (16 + NH - 1) / NH;  // softmax elements per phase B slot
  constexpr int EC = (16 + NC - 1) / NC;  // per phase C slot
  __shared__ __attribute__((aligned(16))) char smem_raw[P::LDS_BYTES];
  __shared__ __attribute__((aligned(16))) float stat[2][2][kBN];  // [buffer][lse*log2e | delta][query]
  lds_char* const smem = (lds_char*)smem_raw;
  auto qb_ = [&](int i) { return smem + i * P::TILE_BYTES; };
  auto gb_ = [&](int i) { return smem + (2 + i) * P::TILE_BYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h_half = lane >> 5;
  int wg = blockIdx.x;
  const int kblk = wg % a.n_tiles;
  wg /= a.n_tiles;
  const int h = wg % a.H, b = a.order_b ? longest_first(a.kv_len, a.B, a.S, wg / a.H) : wg / a.H;
  int n = a.kv_len[b];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  const int64_t bh = (int64_t)b * a.H + h;
  const int key = kblk * kKeysPerWg + wave * 32 + (lane & 31);
  const bool key_in = key < a.S;
  const bool key_ok = key < n;
  const int64_t krow = bh * a.S + key;
  if (kblk * kKeysPerWg >= n || a.Tq == 0) {
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
  // Per-query statistics of query tile t: wave 0 fetches lse, wave 1 delta, one query per
  // lane.  stat_fetch only issues the load (a buffer load over the tile's valid queries, so
  // lanes past Tq read 0 without a branch); stat_value forms the value when it is written to
  // LDS at the end of the iteration, so the load's latency hides behind the whole tile
  // instead of stalling its first slots.
  auto stat_fetch = [&](int t) -> float {
    if (wave_u >= 2) return 0.0f;
    const int valid = min(max(a.Tq - t * kBN, 0), kBN);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc((wave_u == 0 ? lse_bh : del_bh) + (int64_t)t * kBN, (uint32_t)valid * 4);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)lane * 4, 0, 0));
  };
  // (delta is kept negated: the dP chains start from it, see below)
  auto stat_value = [&](int t, float raw) -> float {
    if (wave_u != 0) return -raw;
    return t * kBN + lane < a.Tq ? raw * kLog2e : __builtin_inff();
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
    const float x = stat_value(0, stat_fetch(0));
    if (tid < 128) stat[0][tid >> 6][tid & 63] = x;
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __syncthreads();
  for (int t = 0; t < TQ; ++t) {
    const int cur = t & 1;
    const lds_char* qt_ = qb_(cur);
    const lds_char* gt_ = gb_(cur);
    // past the last tile the resources are empty: the loads zero-fill a buffer never read
    const __amdgpu_buffer_rsrc_t q_rs = q_tile(t + 1), g_rs = g_tile(t + 1);
    const float next_raw = stat_fetch(t + 1);
    f32x16 s[2], dp[2];
    u32x4 ppk[4], dpk[4];
    float p8[8], d8[8];
    f32x4 Lq[2];  // lse of four queries, a ring of two groups
    auto stat4 = [&](int g, int which) {  // group g of 4 queries: 8 g' + 4 h + i within half g / 4
      const int q0 = 32 * (g >> 2) + 8 * (g & 3) + 4 * h_half;
      return *reinterpret_cast<const f32x4*>(&stat[cur][which][q0]);
    };
    // the -delta block of half hf in the register order of a dP block: each dP chain starts
    // from it, so that it yields dP - delta
    auto neg_delta16 = [&](int hf) {
      f32x16 r;
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const f32x4 x = stat4(4 * hf + g, 1);
#pragma unroll
        for (int i = 0; i < 4; ++i) r[4 * g + i] = x[i];
      }
      return r;
    };
    f32x16 nd = neg_delta16(0);
    auto frag_ab = [&](int hf, int j) {  // j even: S (A = Q rows), odd: dP (A = dO rows)
      return P::k_frag((j & 1) ? gt_ : qt_, kbase, 2 * (j >> 1) + hf);
    };
    auto mfma_ab = [&](int hf, int j, bf16x8 fr) {
      const int kk = j >> 1;
      f32x16& d = (j & 1) ? dp[hf] : s[hf];
      if (kk == 0) {
        if (j & 1) mfma_vgpr_from(d, fr, vf.v[0], nd);
        else mfma_vgpr_first(d, fr, kf.v[0]);
      } else {
        mfma_vgpr_acc(d, fr, (j & 1) ? vf.v[kk] : kf.v[kk]);
      }
    };
    // element e (0..15) of half hf: register e of block hf, query 32 hf + 8 (e / 4) + 4 h + e % 4
    auto elem = [&](int hf, int e) {
      const int g = 4 * hf + (e >> 2);
      if ((e & 3) == 0 && (e >> 2) + 1 < 4) Lq[(g + 1) & 1] = stat4(g + 1, 0);  // the next group of the same half
      const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[hf][e], c, -Lq[g & 1][e & 3]));
      p8[e & 7] = p;
      d8[e & 7] = p * dp[hf][e];  // dp holds dP - delta
      if ((e & 7) == 7) {
        const int ks = 2 * hf + (e >> 3);
        ppk[ks] = u32x4{pack_bf16x2(p8[0], p8[1]), pack_bf16x2(p8[2], p8[3]), pack_bf16x2(p8[4], p8[5]),
                        pack_bf16x2(p8[6], p8[7])};
        dpk[ks] = u32x4{pack_bf16x2(d8[0], d8[1]), pack_bf16x2(d8[2], d8[3]), pack_bf16x2(d8[4], d8[5]),
                        pack_bf16x2(d8[6], d8[7])};
      }
    };
    // slot j of phases C and D: j even -> dV (A = dO^T, B = P), odd -> dK (A = Q^T, B = dS);
    // m = j / 2 walks (16-query step ks = 2 hf + m / (D/32), block db = m % (D/32))
    auto frag_cd = [&](int hf, int j) {
      const int m = j >> 1;
      return P::v_frag((j & 1) ? qt_ : gt_, vbase, (2 * hf + m / (D / 32)) * (D / 32) + m % (D / 32));
    };
    auto mfma_cd = [&](int hf, int j, bf16x8 fr) {
      const int m = j >> 1, db = m % (D / 32), ks = 2 * hf + m / (D / 32);
      if (j & 1) dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr, __builtin_bit_cast(bf16x8, dpk[ks]), dk[db], 0, 0, 0);
      else dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fr, __builtin_bit_cast(bf16x8, ppk[ks]), dv[db], 0, 0, 0);
    };

    bf16x8 fr[R];
#pragma unroll
    for (int i = 0; i < R; ++i) fr[i] = frag_ab(0, i);
    Lq[0] = stat4(0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // phase A: S, dP of queries 0..31, and the next tiles' DMA
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      mfma_ab(0, j, fr[j % R]);
      if (j + R < NH) fr[j % R] = frag_ab(0, j + R);
      else fr[j % R] = frag_ab(1, j + R - NH);
      if (j < 2 * P::DMA_PER_WAVE) {
        if (j < P::DMA_PER_WAVE) P::dma_block(q_rs, qb_(cur ^ 1), wave_u, lane, j);
        else P::dma_block(g_rs, gb_(cur ^ 1), wave_u, lane, j - P::DMA_PER_WAVE);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    nd = neg_delta16(1);  // for the dP chain of phase B
    xdl_result_guard<14>();
    // phase B: S, dP of queries 32..63; P, dS of queries 0..31
#pragma unroll
    for (int j = 0; j < NH; ++j) {
      mfma_ab(1, j, fr[j % R]);
      if (j + R < NH) fr[j % R] = frag_ab(1, j + R);
      else fr[j % R] = frag_cd(0, j + R - NH);
#pragma unroll
      for (int u = 0; u < EB; ++u)
        if (j * EB + u < 16) elem(0, j * EB + u);
      __builtin_amdgcn_sched_barrier(0);
    }
    Lq[0] = stat4(4, 0);  // group 4 opens the second half
    xdl_result_guard<12>();
    // phase C: dV, dK over queries 0..31; P, dS of queries 32..63
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      mfma_cd(0, j, fr[j % R]);
      if (j + R < NC) fr[j % R] = frag_cd(0, j + R);
      else fr[j % R] = frag_cd(1, j + R - NC);
#pragma unroll
      for (int u = 0; u < EC; ++u)
        if (j * EC + u < 16) elem(1, j * EC + u);
      __builtin_amdgcn_sched_barrier(0);
    }
    // phase D: dV, dK over queries 32..63
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      mfma_cd(1, j, fr[j % R]);
      if (j + R < NC) fr[j % R] = frag_cd(1, j + R);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (tid < 128) stat[cur ^ 1][tid >> 6][tid & 63] = stat_value(t + 1, next_raw);
    __builtin_amdgcn_s_waitcnt(0x0F70);
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

// ---------------------------------------------------- dk, dv (pipelined)
// The same computation at one wave per SIMD with the loop software-pipelined
// across tiles:
// iteration t issues S_{t+1} = Q_{t+1} K^T and dP_{t+1} = dO_{t+1} V^T on the
// MFMA pipe while the VALU turns S_t, dP_t into P_t and dS_t, then accumulates
// dV += dO_t^T P_t and dK += Q_t^T dS_t.  Q and dO tiles are triple-buffered
// (t and t+1 are read while t+2 loads), the per-query statistics too.  The
// iteration is written as fixed slots (one MFMA, the operand read a few slots
// ahead, a share of the softmax work and of the next tiles' DMA) separated by
// scheduling fences, as in the D = 256 forward.  The loop always runs an even
// number of identical iterations: a query tile past Tq is zero-filled by its
// (empty) load and its statistics give P = 0, so the spare iteration adds
// nothing, and no straight-line copy of the pipelined body (where the register
// allocator could move a fresh MFMA result with a VALU copy) is ever needed.
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void bwd_dkdv_pipe_kernel(BwdArgs a) {
  using P = Bf16Dma<D>;
  constexpr int kKeysPerWg = 128;
  constexpr int R = 2;                         // operand reads issued this many slots ahead
  constexpr int NS = P::NQ * (kBN / 32);       // MFMAs of S (and of dP) per tile
  constexpr int NA = 2 * NS;                   // phase A slots: S and dP interleaved
  constexpr int NV = (D / 32) * (kBN / 16);    // MFMAs of dV (and of dK) per tile
  constexpr int NB = 2 * NV;                   // phase B slots
  constexpr int NE = kBN / 2;                  // softmax elements per lane per tile
  constexpr int EPS = (NE + NA - 1) / NA;      // softmax elements per phase A slot
  static_assert(NA * EPS >= NE, "softmax elements must fit the slots");
  __shared__ __attribute__((aligned(16))) char smem_raw[6 * P::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) float stat[3][2][kBN];  // [buffer][lse*log2e | delta][query]
  lds_char* const smem = (lds_char*)smem_raw;
  auto qb_ = [&](int i) { return smem + i * P::TILE_BYTES; };        // Q buffers 0..2
  auto gb_ = [&](int i) { return smem + (3 + i) * P::TILE_BYTES; };  // dO buffers 0..2

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h_half = lane >> 5;
  int wg = blockIdx.x;
  const int kblk = wg % a.n_tiles;
  wg /= a.n_tiles;
  const int h = wg % a.H, b = a.order_b ? longest_first(a.kv_len, a.B, a.S, wg / a.H) : wg / a.H;
  int n = a.kv_len[b];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  const int64_t bh = (int64_t)b * a.H + h;
  const int key = kblk * kKeysPerWg + wave * 32 + (lane & 31);
  const bool key_in = key < a.S;
  const bool key_ok = key < n;
  const int64_t krow = bh * a.S + key;
  if (kblk * kKeysPerWg >= n || a.Tq == 0) {
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
  // Per-query statistics of query tile t: wave 0 fetches lse, wave 1 delta, one query per
  // lane.  stat_fetch only issues the load (a buffer load over the tile's valid queries, so
  // lanes past Tq read 0 without a branch); stat_value forms the value when it is written to
  // LDS at the end of the iteration, so the load's latency hides behind the whole tile
  // instead of stalling its first slots.
  auto stat_fetch = [&](int t) -> float {
    if (wave_u >= 2) return 0.0f;
    const int valid = min(max(a.Tq - t * kBN, 0), kBN);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc((wave_u == 0 ? lse_bh : del_bh) + (int64_t)t * kBN, (uint32_t)valid * 4);
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)lane * 4, 0, 0));
  };
  // (delta is kept negated: the dP chains start from it, see below)
  auto stat_value = [&](int t, float raw) -> float {
    if (wave_u != 0) return -raw;
    return t * kBN + lane < a.Tq ? raw * kLog2e : __builtin_inff();
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

  // prologue: tiles 0 and 1 (and their statistics) in LDS, S_0 and dP_0 in registers
  P::dma_tile(q_tile(0), qb_(0), wave_u, lane);
  P::dma_tile(g_tile(0), gb_(0), wave_u, lane);
  P::dma_tile(q_tile(1), qb_(1), wave_u, lane);  // empty past Tq: zero fill
  P::dma_tile(g_tile(1), gb_(1), wave_u, lane);
  {
    const float x0 = stat_value(0, stat_fetch(0));
    const float x1 = stat_value(1, stat_fetch(1));
    if (tid < 128) {
      stat[0][tid >> 6][tid & 63] = x0;
      stat[1][tid >> 6][tid & 63] = x1;
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  __syncthreads();
  // -delta of the four queries of group g (0..7) of a tile's statistics buffer: softmax
  // element e is register e % 16 of block e / 16, query 32 (e / 16) + 8 ((e % 16) / 4) + 4 h + e % 4
  auto neg_delta4 = [&](int buf, int g) {
    const int q0 = 32 * (g >> 2) + 8 * (g & 3) + 4 * h_half;
    return *reinterpret_cast<const f32x4*>(&stat[buf][1][q0]);
  };
  // the -delta block of query block kb (32 queries) of buffer buf, in the register order of
  // a dP block, so that a dP chain starting from it yields dP - delta
  auto neg_delta16 = [&](int buf, int kb) {
    f32x16 r;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = neg_delta4(buf, 4 * kb + g);
#pragma unroll
      for (int i = 0; i < 4; ++i) r[4 * g + i] = x[i];
    }
    return r;
  };
  f32x16 s0[kBN / 32], d0[kBN / 32], s1[kBN / 32], d1[kBN / 32];
  P::scores_vgpr(s0, kf, qb_(0), kbase);
  P::scores_vgpr(d0, vf, gb_(0), kbase);
  xdl_result_guard();
#pragma unroll
  for (int kb = 0; kb < kBN / 32; ++kb) d0[kb] += neg_delta16(0, kb);  // tile 0: dP_0 - delta once here

  auto iteration = [&](int t, f32x16 (&sc)[kBN / 32], f32x16 (&dc)[kBN / 32], f32x16 (&sn)[kBN / 32],
                       f32x16 (&dn)[kBN / 32]) {
    const int bc = t % 3, bn = (t + 1) % 3, bf = (t + 2) % 3;
    const __amdgpu_buffer_rsrc_t q_rs = q_tile(t + 2), g_rs = g_tile(t + 2);
    const float next_raw = stat_fetch(t + 2);
    // this tile's per-query statistics, four queries at a time: softmax element e is register
    // e % 16 of block e / 16, query 32 (e / 16) + 8 ((e % 16) / 4) + 4 h + e % 4
    auto stat4 = [&](int g, int which) {
      const int q0 = 32 * (g >> 2) + 8 * (g & 3) + 4 * h_half;
      return *reinterpret_cast<const f32x4*>(&stat[bc][which][q0]);
    };
    f32x4 Lq[2];  // groups g and g + 1 (ring of two)
    Lq[0] = stat4(0, 0);
    // dP_{t+1} - delta: each chain of the next tile's dP starts from its block of -delta
    f32x16 nd[kBN / 32];
    nd[0] = neg_delta16(bn, 0);
    u32x4 ppk[kBN / 16], dpk[kBN / 16];
    float pe[NE], de[NE];
    bf16x8 fr[R];
#pragma unroll
    for (int i = 0; i < R; ++i) fr[i] = P::k_frag((i & 1) ? gb_(bn) : qb_(bn), kbase, i >> 1);
    bf16x8 tr[R];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      {
        const int j = i >> 1, kb = j & 1, kk = j >> 1;
        f32x16& acc = (i & 1) ? dn[kb] : sn[kb];
        if (kk == 0) {
          if (i & 1) mfma_vgpr_from(acc, fr[i % R], vf.v[0], nd[kb]);
          else mfma_vgpr_first(acc, fr[i % R], kf.v[0]);
        } else {
          mfma_vgpr_acc(acc, fr[i % R], (i & 1) ? vf.v[kk] : kf.v[kk]);
        }
        if (i == 0) nd[1] = neg_delta16(bn, 1);  // for slot 3
        if (i + R < NA) {
          const int ii = i + R;
          fr[i % R] = P::k_frag((ii & 1) ? gb_(bn) : qb_(bn), kbase, ii >> 1);
        }
      }
      if (i >= NA - R) {  // operands of the first phase B slots
        const int ii = i - (NA - R);
        tr[ii] = P::v_frag((ii & 1) ? qb_(bc) : gb_(bc), vbase, ii >> 1);
      }
      // the next tiles' DMA (past the last tile the resource is empty and the loads
      // zero-fill the buffer)
      if (i < P::DMA_PER_WAVE) P::dma_block(q_rs, qb_(bf), wave_u, lane, i);
      else if (i < 2 * P::DMA_PER_WAVE) P::dma_block(g_rs, gb_(bf), wave_u, lane, i - P::DMA_PER_WAVE);
#pragma unroll
      for (int u = 0; u < EPS; ++u) {
        const int e = i * EPS + u;
        if (e < NE) {
          const int kb = e >> 4, r = e & 15, g = e >> 2;
          if ((e & 3) == 0 && g + 1 < NE / 4) Lq[(g + 1) & 1] = stat4(g + 1, 0);  // the next group's lse
          const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c, -Lq[g & 1][e & 3]));
          pe[e] = p;
          de[e] = p * dc[kb][r];  // dc holds dP - delta
          if (e & 1) {
            ppk[e >> 3][(e & 7) >> 1] = pack_bf16x2(pe[e - 1], p);
            dpk[e >> 3][(e & 7) >> 1] = pack_bf16x2(de[e - 1], de[e]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int j = i >> 1, ks = j / (D / 32), db = j % (D / 32);
      if (i & 1) dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr[i % R], __builtin_bit_cast(bf16x8, dpk[ks]), dk[db], 0, 0, 0);
      else dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr[i % R], __builtin_bit_cast(bf16x8, ppk[ks]), dv[db], 0, 0, 0);
      if (i + R < NB) {
        const int ii = i + R;
        tr[i % R] = P::v_frag((ii & 1) ? qb_(bc) : gb_(bc), vbase, ii >> 1);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
    if (tid < 128) stat[bf][tid >> 6][tid & 63] = stat_value(t + 2, next_raw);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // this wave's tile loads have landed
    lds_barrier();
  };

  for (int t = 0; t < TQ; t += 2) {  // an odd TQ ends with one empty tile
    iteration(t, s0, d0, s1, d1);
    iteration(t + 1, s1, d1, s0, d0);
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
