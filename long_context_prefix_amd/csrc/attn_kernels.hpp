// HIP kernels (gfx950 / MI355X) for prefix-masked attention and its split-KV form.
//
// One kernel template computes, for a (b, h, 128-query-row tile[, key chunk])
// workgroup, softmax attention over the key range [lo, hi) where hi <= n_b =
// kv_len[b]: keys at or past n_b are never loaded (their LDS rows are zero
// filled and their scores forced to -inf), which is the prefix-mask /
// k-v-truncation identity of tabfm PR #80 (section Fix).  The softmax is the
// fp32 online (running max / running sum) form, and partials over key chunks
// carry a natural-log LSE so that they can be merged exactly (tabfm PR #81,
// section Sequence-parallel inference).
//
// Wave layout (4 waves, 256 threads; each wave owns 32 query rows).  The two
// contractions are issued transposed so that one lane owns one query row:
//   S^T[key][q] = K Q^T   : A = K tile from LDS, B = Q^T held in registers
//   O^T[d][q]  += V^T P^T : A = V^T tile from LDS, B = P^T straight from the
//                           registers that hold S^T after the softmax.
// With the 32x32 MFMA output layout, lane l holds query row (l % 32) and half
// of the keys of each 32-key block; lanes l and l ^ 32 share a row, so a row
// max or sum is 16 register ops plus one v_permlane32_swap.  The k index of
// the P.V contraction is free to follow the S^T register order; V^T is stored
// in LDS with its key positions permuted to match (bits 2 and 3 of the key
// index swapped), so every MFMA operand is one 16-byte LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lcp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;  // 4 wavefronts of 64
constexpr int kBM = 128;       // query rows per workgroup (32 per wave)
constexpr int kBN = 64;        // keys per tile
constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* kv_len;
  int B, H, Tq, S;
  float scale_log2;  // softmax scale * log2(e): scores are kept in the log2 domain
  int chunk;         // split mode: keys per chunk
  int C;             // split mode: number of chunks
  int n_qtiles;
  void* out;         // final mode: [B,H,Tq,D] in the input dtype
  float* lse;        // final mode: [B,H,Tq] or null
  float* part_out;   // split mode: [B,H,C,Tq,D]
  float* part_lse;   // split mode: [B,H,C,Tq]
};

__device__ __forceinline__ float pair_max(float x) {
  // lanes l and l^32 hold the two halves of one query row
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Key index (within a tile) held by S^T register r of a lane in half h.
__device__ __forceinline__ int st_key(int kb, int r, int h) { return 32 * kb + 8 * (r >> 2) + 4 * h + (r & 3); }

// Position of key j of a tile in the permuted V^T layout (an involution).
__host__ __device__ constexpr int vt_pos(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // round to nearest even (v_cvt_pk_bf16_f32)
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// ---------------------------------------------------------------- bf16 path
// K tile in LDS row-major [kBN][D + 8]; V^T tile [D][kBN + 8] with permuted
// key positions.  The 16-byte row padding puts the 8 lanes of one LDS access
// phase on distinct banks for the K and V^T operand reads.
template <int D>
struct Bf16Path {
  static constexpr int KSTR = D + 8;    // bf16 elements per K row in LDS
  static constexpr int VSTR = kBN + 8;  // bf16 elements per V^T row in LDS
  static constexpr int LDS_BYTES = (kBN * KSTR + D * VSTR) * 2;
  static constexpr int NCH = D / 32;    // 16-byte chunks per thread per tile, for K and for V
  static constexpr int KPT = D / 32;    // keys per thread in the V transpose
  static constexpr int KGRP = kBN / KPT;
  static constexpr int NQ = D / 16;     // Q^T operand registers (8 bf16 each)
  static constexpr bool kIsF32 = false;

  struct QFrag { bf16x8 v[NQ]; };
  struct Stage { u32x4 k[NCH]; u32x4 v[KPT]; };

  __device__ static void load_q(QFrag& f, const uint16_t* qrow, bool valid, int h) {
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (valid) x = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h);
      f.v[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Global -> registers for keys [t0, t0 + nv) of this (b, h); rows >= nv become zero.
  __device__ static void load_tile(Stage& st, const uint16_t* kb, const uint16_t* vb, int64_t t0, int nv, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = tid + kThreads * i;
      int key = c / (D / 8), dg = c % (D / 8);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < nv) x = *reinterpret_cast<const u32x4*>(kb + (t0 + key) * D + dg * 8);
      st.k[i] = x;
    }
    int kgrp = tid % KGRP, dg = tid / KGRP;
#pragma unroll
    for (int e = 0; e < KPT; ++e) {
      int key = vt_pos(kgrp * KPT + e);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (key < nv) x = *reinterpret_cast<const u32x4*>(vb + (t0 + key) * D + dg * 8);
      st.v[e] = x;
    }
  }

  __device__ static void store_tile(const Stage& st, uint16_t* ks, uint16_t* vt, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = tid + kThreads * i;
      int key = c / (D / 8), dg = c % (D / 8);
      *reinterpret_cast<u32x4*>(ks + key * KSTR + dg * 8) = st.k[i];
    }
    int kgrp = tid % KGRP, dg = tid / KGRP;
    // 8 x KPT transpose: row i of the output holds element i of each loaded chunk.
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      uint32_t w[KPT / 2];
#pragma unroll
      for (int t = 0; t < KPT / 2; ++t) {
        uint32_t a = st.v[2 * t][i >> 1], b = st.v[2 * t + 1][i >> 1];
        w[t] = (i & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      uint16_t* dst = vt + (dg * 8 + i) * VSTR + kgrp * KPT;
      if constexpr (KPT == 8) {
        *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
      } else if constexpr (KPT == 4) {
        *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
      } else {
        *reinterpret_cast<uint32_t*>(dst) = w[0];
      }
    }
  }

  // S^T (two 32-key blocks) = K_tile Q^T, fp32 accumulation.
  __device__ static void scores(f32x16 (&s)[kBN / 32], const QFrag& f, const uint16_t* ks, int lane) {
    const int i = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(ks + (32 * kb + i) * KSTR + 16 * kk + 8 * h);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, f.v[kk], s[kb], 0, 0, 0);
      }
    }
  }

  // O^T += V^T P^T with P rounded to bf16 as the MFMA operand.
  __device__ static void accumulate(f32x16 (&o)[D / 32], const f32x16 (&p)[kBN / 32], const uint16_t* vt, int lane) {
    const int i = lane & 31, h = lane >> 5;
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks) {
      const f32x16& pk = p[ks >> 1];
      const int r0 = 8 * (ks & 1);
      u32x4 pw = {pack_bf16x2(pk[r0 + 0], pk[r0 + 1]), pack_bf16x2(pk[r0 + 2], pk[r0 + 3]),
                  pack_bf16x2(pk[r0 + 4], pk[r0 + 5]), pack_bf16x2(pk[r0 + 6], pk[r0 + 7])};
      bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        bf16x8 a = *reinterpret_cast<const bf16x8*>(vt + (32 * db + i) * VSTR + 16 * ks + 8 * h);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb, o[db], 0, 0, 0);
      }
    }
  }

  // Four consecutive output elements (d0..d0+3) of one row.
  __device__ static void store_out4(void* out, int64_t off, float a, float b, float c, float d) {
    u32x2 w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + off) = w;
  }
};

// ---------------------------------------------------------------- fp32 path
// Same wave layout with v_mfma_f32_32x32x2_f32 (exact fp32 products).  The
// A operands need one element per lane, so K stays row-major with an odd row
// stride (conflict-free column reads) and V stays row-major (lanes read
// consecutive d of one key row); no transpose is needed.
template <int D>
struct F32Path {
  static constexpr int KSTR = D + 1;
  static constexpr int LDS_BYTES = (kBN * KSTR + kBN * D) * 4;
  static constexpr int NCH = D / 16;  // 16-byte chunks per thread per tile, for K and for V
  static constexpr int NQ = D / 2;
  static constexpr bool kIsF32 = true;

  struct QFrag { float v[NQ]; };
  struct Stage { f32x4 k[NCH]; f32x4 v[NCH]; };

  __device__ static void load_q(QFrag& f, const float* qrow, bool valid, int h) {
#pragma unroll
    for (int t = 0; t < NQ; ++t) f.v[t] = valid ? qrow[2 * t + h] : 0.0f;
  }

  __device__ static void load_tile(Stage& st, const float* kb, const float* vb, int64_t t0, int nv, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = tid + kThreads * i;
      int key = c / (D / 4), dg = c % (D / 4);
      f32x4 x = {0.f, 0.f, 0.f, 0.f}, y = {0.f, 0.f, 0.f, 0.f};
      if (key < nv) {
        x = *reinterpret_cast<const f32x4*>(kb + (t0 + key) * D + dg * 4);
        y = *reinterpret_cast<const f32x4*>(vb + (t0 + key) * D + dg * 4);
      }
      st.k[i] = x;
      st.v[i] = y;
    }
  }

  __device__ static void store_tile(const Stage& st, float* ks, float* vs, int tid) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      int c = tid + kThreads * i;
      int key = c / (D / 4), dg = c % (D / 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) ks[key * KSTR + dg * 4 + j] = st.k[i][j];
      *reinterpret_cast<f32x4*>(vs + key * D + dg * 4) = st.v[i];
    }
  }

  __device__ static void scores(f32x16 (&s)[kBN / 32], const QFrag& f, const float* ks, int lane) {
    const int i = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) s[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < NQ; ++t) {
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        float a = ks[(32 * kb + i) * KSTR + 2 * t + h];
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, f.v[t], s[kb], 0, 0, 0);
      }
    }
  }

  __device__ static void accumulate(f32x16 (&o)[D / 32], const f32x16 (&p)[kBN / 32], const float* vs, int lane) {
    const int i = lane & 31, h = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = st_key(kb, r, h);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          float a = vs[key * D + 32 * db + i];
          o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[kb][r], o[db], 0, 0, 0);
        }
      }
    }
  }

  __device__ static void store_out4(void* out, int64_t off, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off) = f32x4{a, b, c, d};
  }
};

// ------------------------------------------------------------ the fwd kernel
// Workgroup id -> (query tile, [chunk], head, batch), query tile fastest, so
// the workgroups resident at one time walk the same (b, h) key stream and
// share it through L2.
template <class P, int D, bool PARTIAL>
__device__ __forceinline__ void attn_fwd_body(const FwdArgs& a, char* smem) {
  using Elem = typename std::conditional<P::kIsF32, float, uint16_t>::type;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h_half = lane >> 5;

  int wg = blockIdx.x;
  const int qt = wg % a.n_qtiles;
  wg /= a.n_qtiles;
  int c = 0;
  if (PARTIAL) {
    c = wg % a.C;
    wg /= a.C;
  }
  const int h = wg % a.H;
  const int b = wg / a.H;

  int n = a.kv_len[b];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);
  int lo = 0, hi = n;
  if (PARTIAL) {
    lo = c * a.chunk;
    hi = min(lo + a.chunk, n);
  }

  const int64_t bh = (int64_t)b * a.H + h;
  const int row = qt * kBM + wave * 32 + (lane & 31);
  const bool row_ok = row < a.Tq;
  const int64_t out_row = PARTIAL ? ((bh * a.C + c) * a.Tq + row) : (bh * a.Tq + row);

  if (hi <= lo) {  // no valid key: out = 0, lse = -inf
    if (row_ok) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int rg = 0; rg < 4; ++rg) {
          const int64_t off = out_row * D + 32 * db + 8 * rg + 4 * h_half;
          if (PARTIAL)
            *reinterpret_cast<f32x4*>(a.part_out + off) = f32x4{0.f, 0.f, 0.f, 0.f};
          else
            P::store_out4(a.out, off, 0.f, 0.f, 0.f, 0.f);
        }
      if (h_half == 0) {
        if (PARTIAL) a.part_lse[out_row] = -__builtin_inff();
        else if (a.lse) a.lse[out_row] = -__builtin_inff();
      }
    }
    return;
  }

  const Elem* qrow = reinterpret_cast<const Elem*>(a.q) + (bh * a.Tq + (row_ok ? row : 0)) * D;
  const Elem* kbase = reinterpret_cast<const Elem*>(a.k) + bh * a.S * D;
  const Elem* vbase = reinterpret_cast<const Elem*>(a.v) + bh * a.S * D;
  Elem* ks = reinterpret_cast<Elem*>(smem);
  Elem* vs = ks + kBN * P::KSTR;

  typename P::QFrag qf;
  P::load_q(qf, qrow, row_ok, h_half);

  f32x16 o[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
  float m = -__builtin_inff();  // running max, log2 domain
  float l = 0.0f;               // running sum of 2^(x - m)

  typename P::Stage st;
  P::load_tile(st, kbase, vbase, lo, min(kBN, hi - lo), tid);

  for (int t0 = lo; t0 < hi; t0 += kBN) {
    const int nv = min(kBN, hi - t0);
    __syncthreads();  // previous tile fully consumed
    P::store_tile(st, ks, vs, tid);
    __syncthreads();
    if (t0 + kBN < hi) P::load_tile(st, kbase, vbase, t0 + kBN, min(kBN, hi - t0 - kBN), tid);

    f32x16 s[kBN / 32];
    P::scores(s, qf, ks, lane);

    float mt = -__builtin_inff();
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float x = s[kb][r] * a.scale_log2;
        if (nv < kBN && st_key(kb, r, h_half) >= nv) x = -__builtin_inff();
        s[kb][r] = x;
        mt = fmaxf(mt, x);
      }
    mt = pair_max(mt);
    const float m_new = fmaxf(m, mt);
    const float alpha = __builtin_amdgcn_exp2f(m - m_new);
    m = m_new;
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float p = __builtin_amdgcn_exp2f(s[kb][r] - m_new);
        s[kb][r] = p;
        rs += p;
      }
    l = l * alpha + pair_sum(rs);
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][r] *= alpha;

    P::accumulate(o, s, vs, lane);
  }

  if (!row_ok) return;
  const float inv_l = 1.0f / l;
  const float lse_nat = (m + __builtin_amdgcn_logf(l)) * kLn2;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int64_t off = out_row * D + 32 * db + 8 * rg + 4 * h_half;
      const float x0 = o[db][4 * rg + 0] * inv_l, x1 = o[db][4 * rg + 1] * inv_l;
      const float x2 = o[db][4 * rg + 2] * inv_l, x3 = o[db][4 * rg + 3] * inv_l;
      if (PARTIAL)
        *reinterpret_cast<f32x4*>(a.part_out + off) = f32x4{x0, x1, x2, x3};
      else
        P::store_out4(a.out, off, x0, x1, x2, x3);
    }
  if (h_half == 0) {
    if (PARTIAL) a.part_lse[out_row] = lse_nat;
    else if (a.lse) a.lse[out_row] = lse_nat;
  }
}

template <class P, int D, bool PARTIAL, int WAVES_PER_EU>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void attn_fwd_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[P::LDS_BYTES];
  attn_fwd_body<P, D, PARTIAL>(a, smem);
}

// ------------------------------------------------------------ LSE combine
// One row (b, h, i) is handled by D/4 consecutive threads, each owning four
// consecutive output columns; a 256-thread workgroup covers 1024/D rows.
struct CombineArgs {
  const float* part_out;
  const float* part_lse;
  int64_t rows;  // B * H * Tq
  int C, Tq;
  void* out;
  float* lse;
};

template <int D, bool OUT_F32>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void lse_combine_kernel(CombineArgs a) {
  constexpr int TPR = D / 4;  // threads per row
  const int64_t row = (int64_t)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  if (row >= a.rows) return;
  const int col = (threadIdx.x % TPR) * 4;
  const int64_t bh = row / a.Tq;
  const int i = (int)(row - bh * a.Tq);
  const float* pl = a.part_lse + bh * a.C * a.Tq + i;       // stride Tq between chunks
  const float* po = a.part_out + (bh * a.C * a.Tq + i) * D + col;  // stride Tq*D between chunks

  float mx = -__builtin_inff();
  for (int c = 0; c < a.C; ++c) mx = fmaxf(mx, pl[(int64_t)c * a.Tq]);

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  if (mx != -__builtin_inff()) {
    int c = 0;
    for (; c + 4 <= a.C; c += 4) {
      f32x4 x[4];
      float lc[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        lc[u] = pl[(int64_t)(c + u) * a.Tq];
        x[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)(c + u) * a.Tq * D);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float w = __builtin_amdgcn_exp2f((lc[u] - mx) * kLog2e);
        wsum += w;
        acc += w * x[u];
      }
    }
    for (; c < a.C; ++c) {
      const float w = __builtin_amdgcn_exp2f((pl[(int64_t)c * a.Tq] - mx) * kLog2e);
      wsum += w;
      acc += w * *reinterpret_cast<const f32x4*>(po + (int64_t)c * a.Tq * D);
    }
    acc *= 1.0f / wsum;
  }
  const int64_t off = row * D + col;
  if (OUT_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(a.out) + off) = acc;
  } else {
    u32x2 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(a.out) + off) = w;
  }
  if (a.lse && col == 0) a.lse[row] = (mx == -__builtin_inff()) ? mx : mx + __builtin_amdgcn_logf(wsum) * kLn2;
}

}  // namespace lcp
