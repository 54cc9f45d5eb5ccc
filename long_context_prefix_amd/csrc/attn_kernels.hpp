// HIP kernels (gfx950 / MI355X) for prefix-masked attention and its split-KV form.
//
// One kernel template computes, for a (b, h, 128-query-row tile[, key chunk])
// workgroup, softmax attention over the key range [lo, hi) where hi <= n_b =
// kv_len[b]: keys at or past n_b are never loaded (their LDS rows are zero
// filled and their scores forced to -inf), which is the prefix-mask /
// k-v-truncation identity of tabfm PR #80 (section Fix).  The softmax is an
// fp32 online form with a running sum: the bf16 kernels take a pass's
// probabilities against one reference max per row and run the pass again in
// the rare case that a tile climbs too far past it (PassSoftmax); the fp32
// path moves a running max every tile.  Partials over key chunks carry a
// natural-log LSE so that they can be merged exactly (tabfm PR #81, section
// Sequence-parallel inference).
//
// Wave layout (4 waves, 256 threads; each wave owns 32 query rows).  The two
// contractions are issued transposed so that one lane owns one query row:
//   S^T[key][q] = K Q^T   : A = K tile from LDS, B = Q^T held in registers
//   O^T[d][q]  += V^T P^T : A = V^T tile from LDS, B = P^T straight from the
//                           registers that hold S^T after the softmax.
// With the 32x32 MFMA output layout, lane l holds query row (l % 32) and half
// of the keys of each 32-key block; lanes l and l ^ 32 share a row, so a row
// max or sum is 16 register ops plus one v_permlane32_swap.  The k index of
// the P.V contraction follows the S^T register order.
//
// bf16 inputs: K and V tiles are copied global -> LDS by buffer loads that
// write LDS directly (no staging registers), K operands are 16-byte LDS reads
// and V^T operands come from the transposing LDS read; fp32 inputs use a
// plain register-staged tile loop with fp32 MFMA.
//
// The file also holds the log-sum-exp merge of split-KV partials and the
// device-side prefix-mask detector; the backward kernels, built on the same
// tile layout, are in attn_bwd_kernels.hpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace lcp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr int kThreads = 256;  // 4 wavefronts of 64
constexpr int kBM = 128;       // query rows per workgroup (32 per wave)
constexpr int kBM8 = 256;      // the same with eight waves (see bf16_fwd_dma)
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
  int32_t* counters; // single-launch split mode: [B,H,n_qtiles] arrival counts, zero between launches
  int wg_base;        // workgroups of this part start at blockIdx.x = wg_base (a launch split
  int row_base;       // between two kernels' paths); its query rows start at row_base
  int order_b;        // 1: batch elements are walked longest prefix first (1 < B <= 64)
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

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  // round to nearest even (v_cvt_pk_bf16_f32)
  bf16x2 p = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, p);
}

// Raw buffer resource over [base, base + bytes) (gfx9-family descriptor word 3).
// The arguments are workgroup-uniform; readfirstlane keeps the descriptor in SGPRs (a
// descriptor in VGPRs would need a waterfall loop around every load).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)p);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(p >> 32));
  const uint32_t n = __builtin_amdgcn_readfirstlane(bytes);
  void* b = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(b, (short)0, (int)n, 0x00020000);
}

// S^T accumulation with the accumulator in VGPRs.  With one wave per SIMD the
// compiler gives every MFMA the AGPR form, which would make each score travel
// AGPR -> VGPR (v_accvgpr_read) before the softmax can touch it; written out here
// the score MFMAs keep their result where the VALU reads it, while the O
// accumulator stays in AGPRs.  Because the compiler does not know these are
// MFMAs, their consumers must leave the wait states the hardware requires
// between an XDL result and a VALU read (the fixed-slot schedule below does).
__device__ __forceinline__ void mfma_vgpr_first(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_vgpr_acc(f32x16& d, bf16x8 a, bf16x8 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The first MFMA of a chain that starts from a register block c instead of 0 (c is only
// read, so one block can start many chains).
__device__ __forceinline__ void mfma_vgpr_from(f32x16& d, bf16x8 a, bf16x8 b, const f32x16& c) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %3" : "=&v"(d) : "v"(a), "v"(b), "v"(c));
}

// O^T accumulation for the 64-rows-per-wave kernel (whose register file is full at
// D = 256): the accumulator is kept in AGPRs and the operands in VGPRs by the constraints,
// so the compiler cannot move O between register files around the MFMA.  Any VALU read
// of o (v_accvgpr_read) must leave the XDL wait states.
__device__ __forceinline__ void mfma_agpr_acc(f32x16& o, bf16x8 a, u32x4 b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(o) : "v"(a), "v"(b));
}

// W wait states of s_nop (s_nop N gives N + 1).  Every VALU read of an inline-MFMA result
// must come at least 24 wait states after that MFMA on every path (about twice what a
// 32x32x16 MFMA needs); the build's ISA check proves it on the assembly.  Each guard takes
// the fewest nops that, added to the instructions the schedule already places in between,
// reach that distance, since the nops cost issue cycles on every tile.
template <int W>
__device__ __forceinline__ void xdl_nops() {
  static_assert(W >= 0 && W <= 32, "wait states");
  if constexpr (W >= 8) {
    asm volatile("s_nop 7" ::: "memory");
    xdl_nops<W - 8>();
  } else if constexpr (W == 7) {
    asm volatile("s_nop 6" ::: "memory");
  } else if constexpr (W == 6) {
    asm volatile("s_nop 5" ::: "memory");
  } else if constexpr (W == 5) {
    asm volatile("s_nop 4" ::: "memory");
  } else if constexpr (W == 4) {
    asm volatile("s_nop 3" ::: "memory");
  } else if constexpr (W == 3) {
    asm volatile("s_nop 2" ::: "memory");
  } else if constexpr (W == 2) {
    asm volatile("s_nop 1" ::: "memory");
  } else if constexpr (W == 1) {
    asm volatile("s_nop 0" ::: "memory");
  }
}

// W wait states before the VALU reads of the results of the MFMAs above; the scheduling
// fences keep the compiler from moving work across.
template <int W = 24>
__device__ __forceinline__ void xdl_result_guard() {
  __builtin_amdgcn_sched_barrier(0);
  xdl_nops<W>();
  __builtin_amdgcn_sched_barrier(0);
}

// ------------------------------------------------------- bf16 path, DMA layout
// K and V tiles go global -> LDS with 16-byte buffer loads that write LDS
// directly (lane l of one load fills bytes [16 l, 16 l + 16) of a 1 KB block),
// so no staging registers and no LDS stores are needed.  A tile of kBN keys
// is NBLK blocks of 1 KB, each padded to 1040 bytes; a block holds RPB whole
// key rows.  Which key sits in which block follows from the key's bits
// j = 32 kb + 16 s + 8 g + 4 h + e (see blk_of / row_of) and is chosen so that
//   * the QK^T operand read (ds_read_b128: 16 lanes = 16 consecutive keys of
//     one 32-key block, same column) touches 16 distinct bank groups, and
//   * the transposing V read (ds_read_b64_tr_b16: a group of 16 lanes reads
//     4 keys x 32 bytes, lanes l and l+16 the other 32 bytes of the same keys)
//     covers 256 distinct bytes per 32 lanes,
// and so that every operand address is one per-lane base plus an immediate.
// V is read transposed by the hardware: within a 16-lane group, output lane i,
// element e comes from source lane 4e + i/4, element i%4; source lane 4e + jj
// reads 4 consecutive columns (4 jj ..) of key e, so output lane i receives
// column i of 4 keys -- the A operand of V^T P^T with the keys in k order.
template <int D>
struct Bf16Dma {
  static constexpr int ROWB = D * 2;       // bytes per key row
  static constexpr int RPB = 1024 / ROWB;  // rows per block (2, 4, 8)
  static constexpr int NBLK = kBN / RPB;   // blocks per tile (32, 16, 8)
  static constexpr int BLK = 1040;         // padded block stride
  static constexpr int TILE_BYTES = NBLK * BLK;
  static constexpr int LDS_BYTES = 4 * TILE_BYTES;  // K and V (or Q and dO), two buffers each
  static constexpr int NQ = D / 16;
  static constexpr int LPR = ROWB / 16;    // DMA lanes per row
  static constexpr bool kIsF32 = false;
  static_assert(kBN == 64, "the block layout is written for 64-key tiles");

  struct QFrag { bf16x8 v[NQ]; };

  __host__ __device__ static constexpr int blk_of(int j) {
    const int e = j & 3, h = (j >> 2) & 1, g = (j >> 3) & 1, kb = j >> 5;
    if constexpr (D == 256) return 16 * kb + 4 * e + 2 * g + h;
    else if constexpr (D == 128) return 4 * e + 2 * g + h;
    else return 4 * (e & 1) + 2 * g + h;
  }
  __host__ __device__ static constexpr int row_of(int j) {
    const int e = j & 3, s = (j >> 4) & 1, kb = j >> 5;
    if constexpr (D == 256) return s;
    else if constexpr (D == 128) return 2 * kb + s;
    else return 4 * kb + 2 * s + (e >> 1);
  }
  // LDS byte address (within a tile buffer) of key j, byte column col
  __host__ __device__ static constexpr int addr(int j, int col) { return blk_of(j) * BLK + row_of(j) * ROWB + col; }
  // the key stored in row r of block b (inverse of blk_of / row_of)
  __host__ __device__ static constexpr int key_of(int b, int r) {
    int kb = 0, s = 0, g = 0, h = 0, e = 0;
    h = b & 1;
    g = (b >> 1) & 1;
    if constexpr (D == 256) {
      kb = b >> 4; e = (b >> 2) & 3; s = r;
    } else if constexpr (D == 128) {
      kb = r >> 1; s = r & 1; e = b >> 2;
    } else {
      kb = r >> 2; s = (r >> 1) & 1; e = 2 * (r & 1) + (b >> 2);
    }
    return 32 * kb + 16 * s + 8 * g + 4 * h + e;
  }

  __device__ static void load_q(QFrag& f, const uint16_t* qrow, bool valid, int h) {
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
      u32x4 x = {0u, 0u, 0u, 0u};
      if (valid) x = *reinterpret_cast<const u32x4*>(qrow + 16 * kk + 8 * h);
      f.v[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // Issue this wave's share of one tile's DMA (blocks wave, wave + NW, ... of a workgroup of
  // NW waves).  The resource covers only the tile's valid rows; other lanes write zeros
  // without a fetch.
  static constexpr int DMA_PER_WAVE = NBLK / 4;  // blocks of one tile each of four waves copies

  // One block (the bi-th of this wave's share) of a tile.  Issued as inline asm on
  // purpose: the compiler cannot tell which LDS bytes a direct-to-LDS load writes,
  // so for the builtin it waits for every such load in flight before any later LDS
  // read (stalling each iteration on the next tile's loads).  Here the kernel
  // orders these loads itself: an explicit vmcnt wait and an LDS barrier come
  // before any read of a buffer they fill, and a buffer being filled is never
  // read in the same iteration.  M0 holds the LDS destination; an LDS-DMA load
  // needs one wait state after the SALU write of M0 (the s_nop).  Nothing else in
  // these kernels uses M0.
  // STREAM marks the loads non-temporal, for launches in which every tile is read by
  // one workgroup only (one query tile per head): measured 2.5% faster there, and
  // 6.5% slower where many workgroups re-read the same tiles from L2.
  template <bool STREAM = false, int NW = 4>
  __device__ static void dma_block(__amdgpu_buffer_rsrc_t rs, lds_char* buf, int wave_u, int lane, int bi) {
    const int r = lane / LPR, ch = lane % LPR;
    const int b = wave_u + NW * bi;
    const int j = key_of(b, r);
    const uint32_t lds = (uint32_t)(uintptr_t)(buf + b * BLK);
    const uint32_t voff = (uint32_t)(j * ROWB + ch * 16);
    if constexpr (STREAM)
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds" ::"s"(lds),
                   "v"(voff), "s"(rs)
                   : "m0");
    else
      asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(voff),
                   "s"(rs)
                   : "m0");
  }

  template <bool STREAM = false, int NW = 4>
  __device__ static void dma_tile(__amdgpu_buffer_rsrc_t rs, lds_char* buf, int wave_u, int lane) {
#pragma unroll
    for (int bi = 0; bi < NBLK / NW; ++bi) dma_block<STREAM, NW>(rs, buf, wave_u, lane, bi);
  }

  // per-lane base of the QK^T operand read (key i = lane % 32 of block kb = 0, chunk h)
  __device__ static int k_base(int lane) { return addr(lane & 31, 16 * (lane >> 5)); }
  // per-lane base of the transposing V read (source role: key e of group h, columns 4 jj ..)
  __device__ static int v_base(int lane) {
    const int grp = lane >> 4, s16 = lane & 15;
    const int hv = grp >> 1, dh = grp & 1, e = s16 >> 2, jj = s16 & 3;
    return addr(4 * hv + e, 32 * dh + 8 * jj);
  }

  // S^T (two 32-key blocks) = K_tile Q^T, with the accumulators in VGPRs: at one wave
  // per SIMD the compiler would give the MFMAs AGPR results, which the softmax would
  // have to copy out.  The caller must leave the XDL-to-VALU wait states
  // (xdl_result_guard) before reading s.
  __device__ static void scores_vgpr(f32x16 (&s)[kBN / 32], const QFrag& f, const lds_char* kt, int kbase) {
#pragma unroll
    for (int kk = 0; kk < NQ; ++kk) {
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        const int off = addr(32 * kb, 32 * kk) - addr(0, 0);
        bf16x8 a = *(const __attribute__((address_space(3))) bf16x8*)(kt + kbase + off);
        if (kk == 0) mfma_vgpr_first(s[kb], a, f.v[0]);
        else mfma_vgpr_acc(s[kb], a, f.v[kk]);
      }
    }
  }

  // O^T += V^T P^T; pk[ks] holds P for keys 16 ks .. 16 ks + 15 (S^T register order).
  __device__ static void accumulate(f32x16 (&o)[D / 32], const u32x4 (&pk)[kBN / 16], const lds_char* vt, int vbase) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const lds_char* vb = vt + vbase;
#pragma unroll
    for (int ks = 0; ks < kBN / 16; ++ks) {
      const bf16x8 pb = __builtin_bit_cast(bf16x8, pk[ks]);
      const int kb = ks >> 1, sh = ks & 1;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int off0 = addr(32 * kb + 16 * sh, 64 * db) - addr(0, 0);
        const int off1 = addr(32 * kb + 16 * sh + 8, 64 * db) - addr(0, 0);
        s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + off0));
        s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vb + off1));
        s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), pb, o[db], 0, 0, 0);
      }
    }
  }

  __device__ static void store_out4(void* out, int64_t off, float a, float b, float c, float d) {
    u32x2 w = {pack_bf16x2(a, b), pack_bf16x2(c, d)};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + off) = w;
  }
  // ---- manually ordered iteration halves (sched_barrier fences pin the order) ----
  __device__ static bf16x8 k_frag(const lds_char* kt, int kbase, int i) {
    const int off = addr(32 * (i & 1), 32 * (i >> 1)) - addr(0, 0);
    return *(const __attribute__((address_space(3))) bf16x8*)(kt + kbase + off);
  }
  __device__ static bf16x8 v_frag(const lds_char* vt, int vbase, int i) {
    typedef short s16x4 __attribute__((ext_vector_type(4)));
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
    const int ks = i / (D / 32), db = i % (D / 32);
    const int kb = ks >> 1, sh = ks & 1;
    const int off0 = addr(32 * kb + 16 * sh, 64 * db) - addr(0, 0);
    const int off1 = addr(32 * kb + 16 * sh + 8, 64 * db) - addr(0, 0);
    s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + vbase + off0));
    s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(vt + vbase + off1));
    s16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    return __builtin_bit_cast(bf16x8, a);
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

// ------------------------------------------------------------ the fwd kernels
// Batch element with the r-th longest prefix (equal lengths in index order), for
// 1 < B <= 64, from the device-resident lengths and without a host round trip.
// Packed batches have a different boundary per element (tabfm PR #80, section
// Fix), so workgroups of a long element run for longer: walking the elements
// longest first leaves the short ones for the end of the launch, where they fill
// the gaps instead of one long element running alone.  Lane i < B takes n_i and
// counts the elements ordered before it; the lane whose count is r names the
// element.  The result is wave-uniform.
__device__ __forceinline__ int longest_first(const int32_t* kv_len, int B, int S, int r) {
  const int lane = (int)(threadIdx.x & 63);
  int ni = -1;
  if (lane < B) {
    ni = kv_len[lane];
    ni = ni < 0 ? 0 : (ni > S ? S : ni);
  }
  int rank = 0;
  for (int j = 0; j < B; ++j) {
    const int nj = __builtin_amdgcn_readlane(ni, j);
    rank += (nj > ni || (nj == ni && j < lane)) ? 1 : 0;
  }
  const uint64_t hit = __builtin_amdgcn_ballot_w64(lane < B && rank == r);
  return __builtin_amdgcn_readfirstlane((int)__builtin_ctzll(hit));
}
constexpr int kMaxOrderedBatch = 64;

// Workgroup id -> (query tile, [chunk], head, batch), query tile fastest, so
// the workgroups resident at one time walk the same (b, h) key stream and
// share it through L2.  The batch index is the slowest, in longest-first order
// when order_b is set.
struct Work {
  int b, h, c, lo, hi, row;
  bool row_ok;
  int64_t bh, out_row;
};

// local_row: this lane's row within a query tile of tile_rows rows
template <bool PARTIAL>
__device__ __forceinline__ Work decode(const FwdArgs& a, int tile_rows, int local_row) {
  Work w;
  int wg = (int)blockIdx.x - a.wg_base;
  const int qt = wg % a.n_qtiles;
  wg /= a.n_qtiles;
  w.c = 0;
  if (PARTIAL) {
    w.c = wg % a.C;
    wg /= a.C;
  }
  w.h = wg % a.H;
  w.b = a.order_b ? longest_first(a.kv_len, a.B, a.S, wg / a.H) : wg / a.H;
  int n = a.kv_len[w.b];
  n = n < 0 ? 0 : (n > a.S ? a.S : n);  // out-of-range lengths are clamped, never trusted
  w.lo = 0;
  w.hi = n;
  if (PARTIAL) {
    w.lo = w.c * a.chunk;
    w.hi = min(w.lo + a.chunk, n);
  }
  w.bh = (int64_t)w.b * a.H + w.h;
  w.row = a.row_base + qt * tile_rows + local_row;
  w.row_ok = w.row < a.Tq;
  w.out_row = PARTIAL ? ((w.bh * a.C + w.c) * a.Tq + w.row) : (w.bh * a.Tq + w.row);
  return w;
}

// Epilogue: out = O / l (or the fp32 partial) and lse = ln sum exp.  A row
// without any valid key (o = 0, inv_l = 0, lse = -inf) writes zeros.
template <class P, int D, bool PARTIAL>
__device__ __forceinline__ void write_rows(const FwdArgs& a, const Work& w, const f32x16 (&o)[D / 32], float inv_l,
                                           float lse_nat, int h_half) {
  if (!w.row_ok) return;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int64_t off = w.out_row * D + 32 * db + 8 * rg + 4 * h_half;
      const float x0 = o[db][4 * rg + 0] * inv_l, x1 = o[db][4 * rg + 1] * inv_l;
      const float x2 = o[db][4 * rg + 2] * inv_l, x3 = o[db][4 * rg + 3] * inv_l;
      if (PARTIAL)
        *reinterpret_cast<f32x4*>(a.part_out + off) = f32x4{x0, x1, x2, x3};
      else
        P::store_out4(a.out, off, x0, x1, x2, x3);
    }
  if (h_half == 0) {
    if (PARTIAL) a.part_lse[w.out_row] = lse_nat;
    else if (a.lse) a.lse[w.out_row] = lse_nat;
  }
}

// Partial rows of one wave through LDS: the wave's 32 rows are staged row-major
// (16-byte unit u of row r at unit u ^ (r mod D/4), so that neither the writes,
// one unit per lane in 32 rows, nor the reads, whole rows, meet a bank twice),
// then each store instruction writes 1 KB of consecutive rows.  The rows of a
// workgroup are consecutive in part_out, so the stores cover whole cache lines
// instead of 32-byte pieces of 32 rows, and they are issued at device scope and
// non-temporal (cache policy sc1 nt): written through the XCD's L2 rather than
// left there dirty among the streaming tile loads.  On MI355X this took the
// split-KV partial at the inducing shape from 6.2 to 5.6 ms; whole-line stores
// with the default policy, or 32-byte pieces with any policy, measured no gain.
constexpr int kCpolSc1Nt = 16 | 2;  // buffer-store cache policy bits: sc1 (device scope), nt

template <int D>
__device__ __forceinline__ void write_partial_staged(const FwdArgs& a, const Work& w, const f32x16 (&o)[D / 32],
                                                     float inv_l, float lse_nat, int h_half, lds_char* stage,
                                                     int lane) {
  constexpr int U = D / 4;  // 16-byte units per row
  const int r = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int u = 8 * db + 2 * rg + h_half;
      const f32x4 x = {o[db][4 * rg + 0] * inv_l, o[db][4 * rg + 1] * inv_l, o[db][4 * rg + 2] * inv_l,
                       o[db][4 * rg + 3] * inv_l};
      *reinterpret_cast<__attribute__((address_space(3))) f32x4*>(stage + (r * U + (u ^ (r & (U - 1)))) * 16) = x;
    }
  // the wave's rows [row0, row0 + 32) are rows out0.. of part_out; rows at or past Tq lie
  // outside the resource, so their stores are dropped
  const int row0 = w.row - r;
  const int nrows = min(max(a.Tq - row0, 0), 32);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(a.part_out + (w.out_row - r) * D, (uint32_t)(nrows * D * 4));
#pragma unroll
  for (int k = 0; k < 32 * U / 64; ++k) {
    const int idx = 64 * k + lane, rr = idx / U, c = idx % U;
    const f32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) f32x4*>(
        stage + (rr * U + (c ^ (rr & (U - 1)))) * 16);
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rs, (uint32_t)(idx * 16), 0, kCpolSc1Nt);
  }
  if (h_half == 0 && w.row_ok) a.part_lse[w.out_row] = lse_nat;
}

// The bf16 output rows of one 32-row group through LDS, as write_partial_staged does for
// the fp32 partials: lane (r, h) holds 8 bytes of each 16-byte unit 4 db + rg of row r
// (columns 32 db + 8 rg + 4 h ..), staged row-major with unit u of row r at u ^ (r mod D/8);
// then each store instruction writes 1 KB of consecutive rows (2, 4 or 8 whole rows), at
// device scope and non-temporal, instead of 8-byte pieces of 32 rows.  The 8-byte pieces
// cost 2.6 times the output bytes in HBM writes at the 121k-key ICL shape.
template <int D>
__device__ __forceinline__ void write_out_staged(const FwdArgs& a, const Work& w, const f32x16 (&o)[D / 32],
                                                 float inv_l, float lse_nat, int h_half, lds_char* stage, int lane) {
  constexpr int U = D / 8;  // 16-byte units per row
  const int r = lane & 31;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int rg = 0; rg < 4; ++rg) {
      const int u = 4 * db + rg;
      const u32x2 x = {pack_bf16x2(o[db][4 * rg + 0] * inv_l, o[db][4 * rg + 1] * inv_l),
                       pack_bf16x2(o[db][4 * rg + 2] * inv_l, o[db][4 * rg + 3] * inv_l)};
      *reinterpret_cast<__attribute__((address_space(3))) u32x2*>(stage + (r * U + (u ^ (r & (U - 1)))) * 16 +
                                                                  8 * h_half) = x;
    }
  // the group's rows [row0, row0 + 32) are consecutive rows of out; rows at or past Tq lie
  // outside the resource, so their stores are dropped
  const int row0 = w.row - r;
  const int nrows = min(max(a.Tq - row0, 0), 32);
  const __amdgpu_buffer_rsrc_t rs =
      make_rsrc(reinterpret_cast<uint16_t*>(a.out) + (w.out_row - r) * D, (uint32_t)(nrows * D * 2));
#pragma unroll
  for (int k = 0; k < 32 * U / 64; ++k) {
    const int idx = 64 * k + lane, rr = idx / U, c = idx % U;
    const u32x4 x = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
        stage + (rr * U + (c ^ (rr & (U - 1)))) * 16);
    __builtin_amdgcn_raw_buffer_store_b128(x, rs, (uint32_t)(idx * 16), 0, kCpolSc1Nt);
  }
  if (h_half == 0 && w.row_ok && a.lse) a.lse[w.out_row] = lse_nat;
}

template <class P, int D, bool PARTIAL>
__device__ __forceinline__ void write_empty(const FwdArgs& a, const Work& w, int h_half) {
  f32x16 z[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) z[db] = f32x16{};
  write_rows<P, D, PARTIAL>(a, w, z, 0.0f, -__builtin_inff(), h_half);
}

// Plain tile loop (fp32 inputs): one LDS buffer, register prefetch of the next
// tile, softmax rescaled every tile.
template <class P, int D, bool PARTIAL>
__device__ __forceinline__ void attn_fwd_body(const FwdArgs& a, char* smem) {
  using Elem = float;
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int h_half = lane >> 5;
  const Work w = decode<PARTIAL>(a, kBM, wave * 32 + (lane & 31));
  if (w.hi <= w.lo) {
    write_empty<P, D, PARTIAL>(a, w, h_half);
    return;
  }
  const int lo = w.lo, hi = w.hi;

  const Elem* qrow = reinterpret_cast<const Elem*>(a.q) + (w.bh * a.Tq + (w.row_ok ? w.row : 0)) * D;
  const Elem* kbase = reinterpret_cast<const Elem*>(a.k) + w.bh * a.S * D;
  const Elem* vbase = reinterpret_cast<const Elem*>(a.v) + w.bh * a.S * D;
  Elem* ks = reinterpret_cast<Elem*>(smem);
  Elem* vs = ks + kBN * P::KSTR;

  typename P::QFrag qf;
  P::load_q(qf, qrow, w.row_ok, h_half);

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
  write_rows<P, D, PARTIAL>(a, w, o, 1.0f / l, (m + __builtin_amdgcn_logf(l)) * kLn2, h_half);
}

// Workgroup barrier that orders LDS only: tile loads in flight (vmcnt) are not
// drained, so callers wait for exactly the loads they need before it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Softmax state of one lane of the bf16 kernels, for G query rows (1 in the 32-row kernel,
// 2 in the 64-row kernel), each with half of its keys in this lane.
//
// O is never rescaled inside the tile loop.  All probabilities of a pass are taken
// against one reference per row: the first tile's (scaled) max.  No per-tile max is
// taken either: a tile is checked through the sums that the loop forms anyway.  While a
// lane's sum over a tile stays at or below 2^kSlackLog2, every p of it does too, so the
// tile's scores are at most the reference + kSlackLog2, and the sums cannot overflow (a
// row has fewer than 2^22 keys, so this holds for any V below 2^86).  A tile that breaks
// this marks the pass bad and records its exact max; the workgroup then runs the pass
// again against max(reference + kSlackLog2, recorded maxima), which every score of the
// row is at or below.  O / l is the same softmax either way: only the common scale
// differs.  Natural inputs stay within the slack (a row's scores would have to climb
// 20 log2 units past its first tile's max), so the second pass is rare; the per-tile max
// it replaces cost the 32-row kernel 3% of its time.
constexpr float kSlackLog2 = 20.0f;

template <int G>
struct PassSoftmax {
  float m[G];     // the reference this pass takes probabilities against
  float mtop[G];  // the largest exact max of a tile that broke the slack (or -inf)
  float l[G];     // this lane's partial row sums (lanes l and l^32 are added at the end)
  bool bad = false;  // some tile of this wave broke the slack in this pass
  __device__ __forceinline__ PassSoftmax() {
#pragma unroll
    for (int g = 0; g < G; ++g) m[g] = mtop[g] = -__builtin_inff(), l[g] = 0.f;
  }
  // The reference of the next pass (every score of row g is at or below it).
  __device__ __forceinline__ void next_pass() {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = fmaxf(m[g] + kSlackLog2, mtop[g]);
      mtop[g] = -__builtin_inff();
      l[g] = 0.f;
    }
    bad = false;
  }
};

// Scaled row max of one 32-key score block (this lane's keys, then its partner lane's).
__device__ __forceinline__ float row_max32(const f32x16& s, float c) {
  float mt = fmaxf(s[0], s[1]);
#pragma unroll
  for (int r = 2; r < 16; ++r) mt = fmaxf(mt, s[r]);
  return pair_max(mt) * c;
}
// The same for a 64-key tile (two blocks).
__device__ __forceinline__ float row_max64(const f32x16 (&s)[2], float c) {
  float mt = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = (kb == 0 ? 2 : 0); r < 16; ++r) mt = fmaxf(mt, s[kb][r]);
  return pair_max(mt) * c;
}

// Does any of the NW waves of the workgroup need a second pass?  Every wave calls this
// after its last tile load has landed; flags are NW ints of LDS that no tile load writes.
template <int NW = 4>
__device__ __forceinline__ bool workgroup_redo(volatile __attribute__((address_space(3))) int* flags, bool bad,
                                               int wave, int lane) {
  if (lane == 0) flags[wave] = bad ? 1 : 0;
  __syncthreads();
  int any = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) any |= flags[i];
  const bool redo = any != 0;
  __syncthreads();  // the flags are read before any wave can write them again
  return redo;
}

// bf16 path with direct-to-LDS tiles.  At the top of iteration j the scores
// S_j are in registers and K_{j+1}, V_j are in LDS.  Iteration j starts the DMA
// of K_{j+2} and V_{j+1} into the buffers the previous iteration released,
// issues S_{j+1} = K_{j+1} Q^T on the MFMA pipe while the exponentials of tile j
// run on the VALU (against the pass's reference max, see PassSoftmax), checks
// the tile's sums against the slack, accumulates O += V_j P_j, then waits for
// its DMA and meets the other waves at the one barrier of the iteration.  Scores
// of a tile that holds keys at or past the end are masked to -inf (a rare branch)
// before their exponentials.  The loop runs an even number of iterations, so the last one or
// two take phantom tiles past the end: their DMA zero-fills LDS without a memory
// request and every score is masked, so they add p = 0.  The PV product of the last
// real tile then needs no code of its own (a separate last-tile path made the
// register allocator spill), and the loop body is one pair of iterations whose score
// register sets alternate without copies.
//
// The iteration is written as fixed slots -- one MFMA, the LDS operand read
// for the MFMA kRing slots later, a share of the softmax work and, in the
// first slots, one block of the next tiles' DMA -- separated by sched_barrier
// fences that keep the compiler from regrouping them.  At D = 256 (one wave
// per SIMD) nothing else hides a stall; at D = 128 and 64 (two waves per SIMD)
// the fixed order still measured 4-4.5% faster than the compiler's.
//
// NW = 8 runs the same per-wave code with eight waves (256 query rows) per workgroup, one
// workgroup per CU at two waves per SIMD (D = 128 and 64, fused forward only): every tile
// is loaded once for 256 rows instead of once per 128-row workgroup, each wave issues half
// the DMA, and the LDS left free holds four buffers of K and of V instead of two, so a
// tile load has two iterations to land and only every other iteration ends with the wait
// and the barrier.  Its output bits are those of NW = 4; at D = 128 it is 1.5-2 % faster.
//
// Marks a branch whose body runs rarely (the last tile's mask, the slack check's max): an
// empty volatile asm cannot be executed speculatively, so the compiler keeps the branch
// instead of turning its body into selects computed on every iteration.
__device__ __forceinline__ void rare_path() { asm volatile(""); }

constexpr int kRing = 2;  // LDS operand reads issued this many slots ahead (2..4 measure the same)

// LDS of the 32-row kernel with NW waves: K and V in two (NW = 4) or four (NW = 8) buffers
// each, then one second-pass flag per wave.
template <int D, int NW>
constexpr int dma_kernel_lds_bytes() {
  return 2 * (NW == 8 ? 4 : 2) * Bf16Dma<D>::TILE_BYTES + NW * 4;
}

template <int D, bool PARTIAL, bool STREAM, int NW = 4>
__device__ __forceinline__ void bf16_fwd_dma(const FwdArgs& a, char* smem_generic) {
  using P = Bf16Dma<D>;
  static_assert(NW == 4 || (NW == 8 && !PARTIAL && D <= 128), "eight waves: fused forward at D <= 128");
  constexpr int NB = NW == 8 ? 4 : 2;   // LDS buffers of K and of V
  constexpr int DPW = P::NBLK / NW;     // DMA blocks of one tile per wave
  constexpr int KA = NB == 2 ? 2 : 3;   // iteration j loads K_{j+KA} ...
  constexpr int VA = KA - 1;            // ... and V_{j+VA}
  lds_char* const smem = (lds_char*)smem_generic;
  auto kbuf = [&](int m) { return smem + (m & (NB - 1)) * P::TILE_BYTES; };
  auto vbuf = [&](int m) { return smem + (NB + (m & (NB - 1))) * P::TILE_BYTES; };

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h_half = lane >> 5;
  const Work w = decode<PARTIAL>(a, 32 * NW, wave * 32 + (lane & 31));
  if (w.hi <= w.lo) {
    write_empty<P, D, PARTIAL>(a, w, h_half);
    return;
  }
  const int nkeys = w.hi - w.lo;
  const int T = (nkeys + kBN - 1) / kBN;
  auto nv_of = [&](int t) {
    const int r = nkeys - t * kBN;
    return r < 0 ? 0 : (r > kBN ? kBN : r);
  };
  const uint16_t* qrow = reinterpret_cast<const uint16_t*>(a.q) + (w.bh * a.Tq + (w.row_ok ? w.row : 0)) * D;
  const uint16_t* kg = reinterpret_cast<const uint16_t*>(a.k) + (w.bh * a.S + w.lo) * D;
  const uint16_t* vg = reinterpret_cast<const uint16_t*>(a.v) + (w.bh * a.S + w.lo) * D;
  // resource over the valid rows of tile t only (nothing past n_b is ever addressable)
  auto k_tile = [&](int t) { return make_rsrc(kg + (int64_t)t * kBN * D, (uint32_t)nv_of(t) * (D * 2)); };
  auto v_tile = [&](int t) { return make_rsrc(vg + (int64_t)t * kBN * D, (uint32_t)nv_of(t) * (D * 2)); };

  typename P::QFrag qf;
  P::load_q(qf, qrow, w.row_ok, h_half);
  float c = a.scale_log2;
  if (c < 0.0f) {  // c * (q.k) == |c| * ((-q).k): keep c >= 0 so raw-score maxima are the scaled maxima
    c = -c;
#pragma unroll
    for (int kk = 0; kk < P::NQ; ++kk) {
      u32x4 x = __builtin_bit_cast(u32x4, qf.v[kk]) ^ 0x80008000u;
      qf.v[kk] = __builtin_bit_cast(bf16x8, x);
    }
  }
  // masked keys are -inf scores, and c * -inf must stay -inf: a zero scale is taken as the
  // smallest normal float (every finite score then gives 2^0 = 1 to within fp32 rounding)
  c = fmaxf(c, 1.17549435e-38f);
  const int kbase = P::k_base(lane);
  const int vbase = P::v_base(lane);
  // keys at or past nv of a tile get s = -inf; the key indices come from an opaque copy of
  // the lane's half, so that they are computed in the rare branch instead of being hoisted
  // out of the tile loop into live registers
  auto mask_scores = [&](f32x16 (&sg)[kBN / 32], int nv) {
    int hh = h_half;
    asm volatile("" : "+v"(hh));
#pragma unroll
    for (int kb = 0; kb < kBN / 32; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (st_key(kb, r, hh) >= nv) sg[kb][r] = -__builtin_inff();
  };

  volatile __attribute__((address_space(3))) int* const bad_flag =
      (volatile __attribute__((address_space(3))) int*)(smem + 2 * NB * P::TILE_BYTES);  // one per wave
  f32x16 o[D / 32];
  PassSoftmax<1> sm;
  u32x4 pk[kBN / 16];
  // S_j and S_{j+1}, in two register sets used alternately, so that no MFMA of one
  // iteration has to wait for the reads of the previous iteration's scores
  f32x16 s_cur[kBN / 32], s_alt[kBN / 32];

  // sc holds S_j; S_{j+1} is accumulated into sn.  Iteration j reads K_{j+1} and V_j and
  // loads K_{j+KA} and V_{j+VA} into the buffers of K_{j+KA-NB} and V_{j+VA-NB}, which an
  // earlier iteration read last, before a barrier.  With two buffers every iteration ends
  // with the wait for its loads and the barrier; with four only odd iterations do, and the
  // loads of iterations 2p and 2p + 1 are read by iterations 2p + 2 and 2p + 3.
  auto iteration = [&](int j, f32x16 (&sc)[kBN / 32], f32x16 (&sn)[kBN / 32], auto odd_tag) {
    constexpr bool odd = decltype(odd_tag)::value;  // j is odd
    lds_char* const k_next = kbuf(j + 1);
    lds_char* const v_cur = vbuf(j);
    lds_char* const k_free = kbuf(j + KA);
    lds_char* const v_free = vbuf(j + VA);
    const __amdgpu_buffer_rsrc_t k_rs = k_tile(j + KA), v_rs = v_tile(j + VA);
    {
      constexpr int R = kRing;
      constexpr int NS = P::NQ * (kBN / 32);     // QK^T MFMAs per tile
      constexpr int NV = (D / 32) * (kBN / 16);  // PV MFMAs per tile
      constexpr int EPS = (kBN / 2) / NS;        // softmax elements per QK^T slot
      bf16x8 kf[R], vf[R];
#pragma unroll
      for (int i = 0; i < R; ++i) kf[i] = P::k_frag(k_next, kbase, i);
      const float nm = -sm.m[0];
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      float pe[kBN / 2], xe[kBN / 2];
      __builtin_amdgcn_sched_barrier(0);
      // the QK^T phase, which carries the tile's softmax work, runs at wave priority 1 and
      // the PV phase at 0: with two waves per SIMD the issue arbiter then serves the
      // softmax of one wave ahead of the other wave's PV phase, whose MFMAs keep the
      // matrix pipe busy meanwhile (2-3% faster at D = 128 with two waves per SIMD; no
      // effect at one wave per SIMD)
      __builtin_amdgcn_s_setprio(1);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        const int kb = i % (kBN / 32), kk = i / (kBN / 32);
        if (kk == 0) mfma_vgpr_first(sn[kb], kf[i % R], qf.v[0]);
        else mfma_vgpr_acc(sn[kb], kf[i % R], qf.v[kk]);
        if (i + R < NS) kf[i % R] = P::k_frag(k_next, kbase, i + R);
        if (i >= NS - R) vf[i - (NS - R)] = P::v_frag(v_cur, vbase, i - (NS - R));
        // the tile DMA is spread one block per slot over the first QK^T slots: all of it at
        // once would hold this wave's in-order issue (and the MFMA pipe) behind the loads
        if (i < 2 * DPW) {
          if (i < DPW) P::template dma_block<STREAM, NW>(k_rs, k_free, wave_u, lane, i);
          else P::template dma_block<STREAM, NW>(v_rs, v_free, wave_u, lane, i - DPW);
        }
#pragma unroll
        for (int t = 0; t < EPS; ++t) {
          // element e (register e % 16 of S^T block e / 16) is staged over three steps so
          // that no instruction waits on the one just before it: the fma of element e + 2,
          // the exp2 of element e + 1, then the sum and bf16 pack of element e
          const int e = i * EPS + t;
          if (e == 0) {
            xe[0] = __builtin_fmaf(sc[0][0], c, nm);
            xe[1] = __builtin_fmaf(sc[0][1], c, nm);
            pe[0] = __builtin_amdgcn_exp2f(xe[0]);
          }
          if (e + 2 < kBN / 2) xe[e + 2] = __builtin_fmaf(sc[(e + 2) >> 4][(e + 2) & 15], c, nm);
          if (e + 1 < kBN / 2) pe[e + 1] = __builtin_amdgcn_exp2f(xe[e + 1]);
          acc[e & 3] += pe[e];
          if (e & 1) pk[e >> 3][(e & 7) >> 1] = pack_bf16x2(pe[e - 1], pe[e]);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // the tile's sum; past the slack, record the tile's exact max (rare: the scores are
      // still in sc) and mark the pass
      const float sum = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      sm.l[0] += sum;
      if (__builtin_amdgcn_ballot_w64(!(sum <= __builtin_exp2f(kSlackLog2))) != 0) {
        rare_path();
        sm.bad = true;
        sm.mtop[0] = fmaxf(sm.mtop[0], row_max64(sc, c));
      }
      // the scores were written by MFMAs the compiler does not see as such; the work
      // scheduled since the last of them already keeps the VALU reads of S_{j+1} below
      // the 24 wait states clear of it (the build's ISA check proves it), so no nops
      __builtin_amdgcn_sched_barrier(0);
      if (nv_of(j + 1) < kBN) {
        rare_path();
        mask_scores(sn, nv_of(j + 1));
      }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_setprio(0);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int ks = i / (D / 32), db = i % (D / 32);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[i % R], __builtin_bit_cast(bf16x8, pk[ks]), o[db], 0, 0, 0);
        if (i + R < NV) vf[i % R] = P::v_frag(v_cur, vbase, i + R);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (NB == 2 || odd) {
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads so far have landed
      lds_barrier();
    }
  };

  // one pass over the keys; a second runs only if the first marked a row bad (see PassSoftmax)
  const int T2 = (T + 1) & ~1;
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    P::template dma_tile<STREAM, NW>(k_tile(0), kbuf(0), wave_u, lane);
    P::template dma_tile<STREAM, NW>(v_tile(0), vbuf(0), wave_u, lane);
    P::template dma_tile<STREAM, NW>(k_tile(1), kbuf(1), wave_u, lane);
    if constexpr (NB == 4) {  // the first pair of iterations reads K_1, K_2, V_0 and V_1
      P::template dma_tile<STREAM, NW>(k_tile(2), kbuf(2), wave_u, lane);
      P::template dma_tile<STREAM, NW>(v_tile(1), vbuf(1), wave_u, lane);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads have landed in LDS
    __syncthreads();
    // S_0, with the loop's register form of the score MFMAs
#pragma unroll
    for (int kk = 0; kk < P::NQ; ++kk)
#pragma unroll
      for (int kb = 0; kb < kBN / 32; ++kb) {
        const bf16x8 kf = P::k_frag(kbuf(0), kbase, (kBN / 32) * kk + kb);
        if (kk == 0) mfma_vgpr_first(s_cur[kb], kf, qf.v[0]);
        else mfma_vgpr_acc(s_cur[kb], kf, qf.v[kk]);
      }
    xdl_nops<24>();  // XDL result -> VALU read (row max below)
    __syncthreads();  // every wave is done with K_0 before its buffer is refilled
    if (nv_of(0) < kBN) mask_scores(s_cur, nv_of(0));
    if (pass == 0) sm.m[0] = row_max64(s_cur, c);  // the first tile's max is the first pass's reference

    // iterations 0 .. T2 - 1, T2 = T rounded up to even: iteration j adds PV_j and takes the
    // scores of tile j + 1 (phantom tiles at or past T are all masked)
    for (int j = 0; j < T2; j += 2) {
      iteration(j, s_cur, s_alt, std::false_type{});
      iteration(j + 1, s_alt, s_cur, std::true_type{});
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no tile load may still be writing LDS when the pass ends
    if (!workgroup_redo<NW>(bad_flag, sm.bad, wave, lane) || pass > 0) break;
    sm.next_pass();
  }

  const float l = pair_sum(sm.l[0]);
  const float lse_nat = (sm.m[0] + __builtin_amdgcn_logf(l)) * kLn2;
  if constexpr (PARTIAL && STREAM) {
    static_assert(NW * 32 * D * 4 <= 2 * NB * P::TILE_BYTES, "the waves' partial rows fit the tile buffers");
    lds_barrier();  // every wave is done with the last V tile: the buffers take the partial rows
    write_partial_staged<D>(a, w, o, 1.0f / l, lse_nat, h_half, smem + wave * (32 * D * 4), lane);
  } else if constexpr (!PARTIAL) {
    static_assert(NW * 32 * D * 2 <= 2 * NB * P::TILE_BYTES, "the waves' output rows fit the tile buffers");
    lds_barrier();  // every wave is done with the last V tile: the buffers take the output rows
    write_out_staged<D>(a, w, o, 1.0f / l, lse_nat, h_half, smem + wave * (32 * D * 2), lane);
  } else {
    write_rows<P, D, PARTIAL>(a, w, o, 1.0f / l, lse_nat, h_half);
  }
}

// ------------------------------------ bf16, D = 256 and 128, 64 rows per wave
// The same contractions with each wave holding two 32-row groups of queries
// (64 rows, 256 per workgroup) over 32-key tiles.  Every K operand read and
// every transposed V read then feeds two MFMAs (one per group), so the LDS
// operand traffic and the tile DMA per MFMA are half those of bf16_fwd_dma,
// whose D = 256 form is bound by LDS bandwidth rather than by the MFMA pipe.
// At D = 256 the register file holds it only just: O of both groups takes all
// 256 AGPRs, Q of both groups 128 VGPRs.  The tiles come from the 64-key layout
// of Bf16Dma<D> (see WideLayout).  At D = 256 the host takes it for launches
// whose workgroups fill the GPU's waves better this way (its tiles are twice
// as tall, so a last, partly filled wave costs more); the rest keep the 32-row
// kernel.  At D = 128 it is as fast as the 32-row kernel and runs only when
// forced: with half the MFMAs per 32-key tile, its single wave per SIMD waits on
// the softmax VALU work.
constexpr int kBMW = 256;  // query rows per workgroup (64 per wave)
constexpr int kBNW = 32;   // keys per tile

template <int D>
struct WideLayout;

// D = 256: a 32-key tile is the first 16 blocks of the 64-key layout of Bf16Dma<256>
// (keys 0..31), so the operand reads and the DMA are those of that layout.
template <>
struct WideLayout<256> {
  using P = Bf16Dma<256>;
  static constexpr int SUB = 1;                        // 32-key tiles per DMA tile
  static constexpr int NBUF = 4;                       // buffers for K, and for V
  static constexpr int TILE_BYTES = 16 * P::BLK;
  static constexpr int FLAGS = 2 * NBUF * TILE_BYTES;  // K and V buffers; then 4 flags
  static constexpr int LDS_BYTES = FLAGS + 4 * 4;
  static constexpr int DMA_PER_WAVE = 4;            // 16 blocks per tile over 4 waves
  static constexpr int HALF_OFF = 0;                // unused: one 32-key tile per buffer
  static_assert(P::key_of(15, 1) < kBNW && P::blk_of(kBNW - 1) < 16, "keys 0..31 fill blocks 0..15");

  // the lane's part of the DMA offset (row lane / 32, chunk lane % 32), one VGPR for every block
  __device__ static uint32_t dma_arg(int lane) { return (uint32_t)((lane >> 5) * 16 * (256 * 2) + (lane & 31) * 16); }

  // Block b = wave + 4 bi of a tile, as Bf16Dma<256>::dma_block.  The block's part of the
  // global offset, 512 key_of(b, 0), is added into a temporary inside the asm so that no
  // per-block offset stays live, and so that the whole offset is the VGPR offset that the
  // buffer range check sees.
  template <bool STREAM>
  __device__ static void dma_block(__amdgpu_buffer_rsrc_t rs, lds_char* buf, int wave_u, uint32_t voff, int bi) {
    const int b = wave_u + 4 * bi;
    const uint32_t lds = (uint32_t)(uintptr_t)(buf + b * P::BLK);
    const uint32_t boff = (uint32_t)(P::key_of(b, 0) * P::ROWB);
    uint32_t t;
    if constexpr (STREAM)
      asm volatile(
          "v_add_u32 %0, %2, %1\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %4, 0 offen nt lds"
          : "=&v"(t)
          : "v"(voff), "s"(boff), "s"(lds), "s"(rs)
          : "m0");
    else
      asm volatile(
          "v_add_u32 %0, %2, %1\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\tbuffer_load_dwordx4 %0, %4, 0 offen lds"
          : "=&v"(t)
          : "v"(voff), "s"(boff), "s"(lds), "s"(rs)
          : "m0");
  }
};

// D = 128: the DMA moves whole 64-key tiles of the Bf16Dma<128> layout, each holding two
// 32-key tiles.  Keys 32..63 of that layout sit two rows below keys 0..31 in the same
// blocks, so every operand address of the second 32-key tile is the first's plus 512
// bytes (HALF_OFF), with the same bank pattern.
template <>
struct WideLayout<128> {
  using P = Bf16Dma<128>;
  static constexpr int SUB = 2;
  static constexpr int NBUF = 2;
  static constexpr int TILE_BYTES = P::TILE_BYTES;
  static constexpr int FLAGS = 2 * NBUF * TILE_BYTES;
  static constexpr int LDS_BYTES = FLAGS + 4 * 4;
  static constexpr int DMA_PER_WAVE = P::DMA_PER_WAVE;
  static constexpr int HALF_OFF = 2 * P::ROWB;
  static_assert(P::addr(32, 0) - P::addr(0, 0) == HALF_OFF && P::addr(63, 0) - P::addr(31, 0) == HALF_OFF,
                "keys 32..63 sit HALF_OFF bytes past keys 0..31");

  __device__ static uint32_t dma_arg(int lane) { return (uint32_t)lane; }
  template <bool STREAM>
  __device__ static void dma_block(__amdgpu_buffer_rsrc_t rs, lds_char* buf, int wave_u, uint32_t lane, int bi) {
    P::template dma_block<STREAM>(rs, buf, wave_u, (int)lane, bi);
  }
};

// Rows of group 1 sit 32 below those of group 0.
__device__ __forceinline__ Work next_group(const FwdArgs& a, Work w) {
  w.row += 32;
  w.out_row += 32;
  w.row_ok = w.row < a.Tq;
  return w;
}

// XDL wait states before a VALU read of an O tile written by inline MFMAs: the tile is an
// operand of the asm, so no read of it -- the compiler's own register copies included --
// can be placed before the wait.
__device__ __forceinline__ void o_result_guard(f32x16& o) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+a"(o));
}
// The same for two score blocks before their first VALU read (W wait states of nops,
// then an empty asm that takes the blocks as operands).
template <int W>
__device__ __forceinline__ void s_result_guard(f32x16& s0, f32x16& s1) {
  __builtin_amdgcn_sched_barrier(0);
  xdl_nops<W>();
  asm volatile("" : "+v"(s0), "+v"(s1));
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, bool PARTIAL, bool STREAM>
__device__ __forceinline__ void bf16_fwd_wide(const FwdArgs& a, char* smem_generic) {
  using P = Bf16Dma<D>;
  using L = WideLayout<D>;
  constexpr int SUB = L::SUB;         // 32-key tiles per DMA tile (1 at D = 256, 2 at D = 128)
  constexpr int NF = P::NQ;           // K fragments (and V fragments) per 32-key tile: D / 16
  constexpr int SPE = 2 * NF / 16;    // slots per softmax element: 2 at D = 256, 1 at D = 128
  constexpr int NOB = D / 32;         // O blocks per group
  constexpr int TK = kBNW * SUB;      // keys per DMA tile
  lds_char* const smem = (lds_char*)smem_generic;
  // buffer of DMA tile m: K in the first NBUF tile slots, V in the next NBUF
  static_assert((L::NBUF & (L::NBUF - 1)) == 0, "a power of two buffers");
  auto kb = [&](int m) { return smem + (m & (L::NBUF - 1)) * L::TILE_BYTES; };
  auto vb = [&](int m) { return smem + (L::NBUF + (m & (L::NBUF - 1))) * L::TILE_BYTES; };
  volatile __attribute__((address_space(3))) int* const bad_flag =
      (volatile __attribute__((address_space(3))) int*)(smem + L::FLAGS);  // one per wave
  static_assert(L::FLAGS >= 2 * L::NBUF * L::TILE_BYTES && L::FLAGS + 4 * (int)sizeof(int) <= L::LDS_BYTES,
                "the flags sit past the tile buffers, inside the allocation");

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const int h_half = lane >> 5;
  Work w[2];
  w[0] = decode<PARTIAL>(a, kBMW, wave * 64 + (lane & 31));
  w[1] = next_group(a, w[0]);
  if (w[0].hi <= w[0].lo) {
    write_empty<P, D, PARTIAL>(a, w[0], h_half);
    write_empty<P, D, PARTIAL>(a, w[1], h_half);
    return;
  }
  const uint32_t dma_voff = L::dma_arg(lane);
  const int nkeys = w[0].hi - w[0].lo;
  const int T = (nkeys + kBNW - 1) / kBNW;  // 32-key tiles
  auto nv_of = [&](int t) {
    const int r = nkeys - t * kBNW;
    return r < 0 ? 0 : (r > kBNW ? kBNW : r);
  };
  auto nd_of = [&](int m) {  // valid keys of DMA tile m
    const int r = nkeys - m * TK;
    return r < 0 ? 0 : (r > TK ? TK : r);
  };
  const uint16_t* kg = reinterpret_cast<const uint16_t*>(a.k) + (w[0].bh * a.S + w[0].lo) * D;
  const uint16_t* vg = reinterpret_cast<const uint16_t*>(a.v) + (w[0].bh * a.S + w[0].lo) * D;
  // resources over the valid rows of DMA tile m only
  auto k_tile = [&](int m) { return make_rsrc(kg + (int64_t)m * TK * D, (uint32_t)nd_of(m) * (D * 2)); };
  auto v_tile = [&](int m) { return make_rsrc(vg + (int64_t)m * TK * D, (uint32_t)nd_of(m) * (D * 2)); };
  auto dma = [&](__amdgpu_buffer_rsrc_t rs, lds_char* buf) {
#pragma unroll
    for (int bi = 0; bi < L::DMA_PER_WAVE; ++bi) L::template dma_block<STREAM>(rs, buf, wave_u, dma_voff, bi);
  };

  typename P::QFrag qf[2];
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const uint16_t* qrow =
        reinterpret_cast<const uint16_t*>(a.q) + (w[g].bh * a.Tq + (w[g].row_ok ? w[g].row : 0)) * D;
    P::load_q(qf[g], qrow, w[g].row_ok, h_half);
  }
  float c = a.scale_log2;
  if (c < 0.0f) {  // c * (q.k) == |c| * ((-q).k): keep c >= 0 so raw-score maxima are the scaled maxima
    c = -c;
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int kk = 0; kk < P::NQ; ++kk) {
        u32x4 x = __builtin_bit_cast(u32x4, qf[g].v[kk]) ^ 0x80008000u;
        qf[g].v[kk] = __builtin_bit_cast(bf16x8, x);
      }
  }
  // masked keys are -inf scores, and c * -inf must stay -inf: a zero scale is taken as the
  // smallest normal float (every finite score then gives 2^0 = 1 to within fp32 rounding)
  c = fmaxf(c, 1.17549435e-38f);
  const int kbase = P::k_base(lane);
  const int vbase = P::v_base(lane);

  f32x16 o[2][D / 32];
  PassSoftmax<2> sm;
  // Scores of the tile in flight: group 0 has one register block, group 1 two (s1a, s1b),
  // used in alternate iterations, so that group 1's exponentials of tile j run beside the
  // QK^T MFMAs of tile j + 1 while group 0's run beside the PV MFMAs: each phase carries
  // half of the softmax.
  f32x16 s0, s1a, s1b;
  u32x4 p0a[2], p0b[2];  // P of group 0 (keys 16 ks .. in [ks]): two sets, used alternately
  u32x4 p1[2];           // P of group 1
  constexpr int R = 4;  // LDS operand reads issued this many fragments ahead (2 and 3 measure 0.5% slower)

  // Exponentials of one score block sg (group g) into pk, one element r per call, staged so
  // that no instruction waits on the one just before it: the fma of element r + 2, the exp2
  // of r + 1, then the fp32 sum of r and the bf16 pack of r - 1 and r.
  // part 0 issues the exp2 (a quarter-rate instruction) in a slot of its own, part 1 the
  // fma, the sum and the pack; part 2 both.
  auto exp_slot = [&](const f32x16& sg, int g, int r, u32x4 (&pk)[2], float (&xe)[16], float (&pe)[16],
                      float& acc, int part) {
    auto fma_of = [&](int k) { return __builtin_fmaf(sg[k], c, -sm.m[g]); };
    if (part != 1) {
      if (r == 0) {
        xe[0] = fma_of(0);
        xe[1] = fma_of(1);
        pe[0] = __builtin_amdgcn_exp2f(xe[0]);
      }
      if (r + 1 < 16) pe[r + 1] = __builtin_amdgcn_exp2f(xe[r + 1]);
    }
    if (part != 0) {
      if (r + 2 < 16) xe[r + 2] = fma_of(r + 2);
      acc += pe[r];
      if (r & 1) {
        uint32_t d = pack_bf16x2(pe[r - 1], pe[r]);
        asm volatile("" : "+v"(d));  // keeps the pack in this slot (it is used only later)
        pk[r >> 3][(r & 7) >> 1] = d;
      }
    }
  };
  // After a block's exponentials: add the sum to l, and if a lane's sum broke the slack,
  // record the tile's exact scaled max (rare; the scores are still in sg) and mark the pass.
  auto exp_end = [&](const f32x16& sg, int g, float acc) {
    sm.l[g] += acc;
    if (__builtin_amdgcn_ballot_w64(!(acc <= __builtin_exp2f(kSlackLog2))) != 0) {
      rare_path();
      sm.bad = true;
      sm.mtop[g] = fmaxf(sm.mtop[g], row_max32(sg, c));
    }
  };
  // keys at or past nv in a tile count as -inf: p = 2^-inf = 0 (c > 0).  The key indices
  // come from an opaque copy of the lane's half, so that they are computed here (rarely)
  // instead of being hoisted out of the tile loop into 16 live registers.
  auto mask_scores = [&](f32x16& sg0, f32x16& sg1, int nv) {
    int hh = h_half;
    asm volatile("" : "+v"(hh));
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (st_key(0, r, hh) >= nv) {
        sg0[r] = -__builtin_inff();
        sg1[r] = -__builtin_inff();
      }
  };

  // Iteration j.  At its top: group 0 of P_j in p0c, group 1 of S_j in s1c, K_{j+1} and V_j
  // in LDS.
  //  * Phase X, 32 QK^T slots (K fragment kk, group g): S_{j+1} = K_{j+1} Q^T into s0 and
  //    s1n, each K fragment feeding both groups; beside the odd slots, group 1 of S_j (s1c)
  //    goes to P (p1); beside the first even slots, the DMA of K_{j+2} and V_{j+1}.
  //  * Phase Y, 32 PV slots (V fragment, group): O += V_j P_j, each V fragment feeding both
  //    groups; beside the odd slots, group 0 of S_{j+1} goes to P (p0n).  S_{j+1} is masked
  //    first when it holds keys past n.
  // Then the DMA wait and the one barrier.
  auto iteration = [&](int j, auto odd_tag, f32x16& s1c, f32x16& s1n, u32x4 (&p0c)[2], u32x4 (&p0n)[2]) {
    constexpr bool odd = decltype(odd_tag)::value;  // j is odd
    const lds_char* k_next;  // K_{j+1}
    const lds_char* v_cur;   // V_j
    // this iteration's DMA: one tile into buffer d0_buf (and, with one 32-key tile per DMA
    // tile, a second into d1_buf)
    lds_char* d0_buf;
    lds_char* d1_buf = nullptr;
    __amdgpu_buffer_rsrc_t d0_rs, d1_rs;
    if constexpr (SUB == 1) {
      // four buffers each, and a barrier after odd iterations only: iteration j loads
      // K_{j+3} and V_{j+2}, into the buffers of K_{j-1} and V_{j-2}, which iteration j - 2
      // read last (a barrier ends iteration j - 2 or j - 1); the loads of iterations 2p and
      // 2p + 1 are waited for at the barrier that ends 2p + 1, before iterations 2p + 2 and
      // 2p + 3 read them
      k_next = kb(j + 1);
      v_cur = vb(j);
      d0_buf = kb(j + 3);
      d1_buf = vb(j + 2);
      d0_rs = k_tile(j + 3);
      d1_rs = v_tile(j + 2);
    } else {
      // j = 2M or 2M + 1.  K_{j+1} is half (j + 1) & 1 of DMA tile (j + 1) / 2, V_j half j & 1
      // of DMA tile M.  An even iteration loads V tile M + 1 (into the buffer of V tile M - 1,
      // last read by iteration 2M - 1), an odd one K tile M + 2 (into that of K tile M, last
      // read by iteration 2M): each load has two iterations to land.
      const int M = j >> 1;
      lds_char* const kM = kb(M);
      lds_char* const kM1 = kb(M + 1);
      lds_char* const vM = vb(M);
      lds_char* const vM1 = vb(M + 1);
      if (odd) {
        k_next = kM1;
        v_cur = vM + L::HALF_OFF;
        d0_buf = kM;
        d0_rs = k_tile((j >> 1) + 2);
      } else {
        k_next = kM + L::HALF_OFF;
        v_cur = vM;
        d0_buf = vM1;
        d0_rs = v_tile((j >> 1) + 1);
      }
      d1_rs = d0_rs;  // unused
    }
    const int nv = nv_of(j + 1);
    bf16x8 kf[R], vf[R];
    // in order, each behind a fence: the first MFMA then waits for the first read only
    // (the LDS counter counts in issue order)
#pragma unroll
    for (int i = 0; i < R; ++i) {
      kf[i] = P::k_frag(k_next, kbase, 2 * i);
      __builtin_amdgcn_sched_barrier(0);
    }
    {
      float xe[16], pe[16], acc = 0.f;
      // The group-1 softmax runs LAG slots behind the MFMAs: the first LAG slots carry none,
      // and the last LAG slots' share runs after the loop, between the last score MFMA and
      // the first VALU read of S_{j+1} below, where it stands in for most of the wait states
      // that read needs (7 nops are left; 13 nops in place of the lag measured 0.7 % slower).
      constexpr int LAG = 4;
#pragma unroll
      for (int i = 0; i < 2 * NF; ++i) {
        const int kk = i >> 1, g = i & 1;
        f32x16& sg = g == 0 ? s0 : s1n;
        // the slot's share of the softmax goes before its MFMA, so that the VALU work fills the
        // time the operand read has to land before the MFMA waits for it (0.5-1% faster on
        // most of the GPUs measured)
        if (i >= LAG) {
          const int e = i - LAG;
          exp_slot(s1c, 1, e / SPE, p1, xe, pe, acc, SPE == 1 ? 2 : e % SPE);
        }
        if (kk == 0) mfma_vgpr_first(sg, kf[kk % R], qf[g].v[0]);
        else mfma_vgpr_acc(sg, kf[kk % R], qf[g].v[kk]);
        if (g == 1 && kk + R < NF) kf[kk % R] = P::k_frag(k_next, kbase, 2 * (kk + R));
        if (i >= 2 * NF - R) vf[i - (2 * NF - R)] = P::v_frag(v_cur, vbase, i - (2 * NF - R));
        if (g == 0) {
          if (kk < L::DMA_PER_WAVE) L::template dma_block<STREAM>(d0_rs, d0_buf, wave_u, dma_voff, kk);
          else if (SUB == 1 && kk < 2 * L::DMA_PER_WAVE)
            L::template dma_block<STREAM>(d1_rs, d1_buf, wave_u, dma_voff, kk - L::DMA_PER_WAVE);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
#pragma unroll
      for (int e = 2 * NF - LAG; e < 2 * NF; ++e) {
        exp_slot(s1c, 1, e / SPE, p1, xe, pe, acc, SPE == 1 ? 2 : e % SPE);
        __builtin_amdgcn_sched_barrier(0);
      }
      exp_end(s1c, 1, acc);
    }
    // the scores were written by MFMAs the compiler does not see as such: keep the VALU
    // reads of S_{j+1} below clear of the last of them
    s_result_guard<7>(s0, s1n);
    if (nv < kBNW) {
      rare_path();
      mask_scores(s0, s1n, nv);
    }
    __builtin_amdgcn_sched_barrier(0);
    {
      float xe[16], pe[16], acc = 0.f;
#pragma unroll
      for (int i = 0; i < 2 * NF; ++i) {
        const int vi = i >> 1, g = i & 1;  // V fragment vi: keys 16 (vi / NOB) .., columns 32 (vi % NOB) ..
        exp_slot(s0, 0, i / SPE, p0n, xe, pe, acc, SPE == 1 ? 2 : i % SPE);
        mfma_agpr_acc(o[g][vi % NOB], vf[vi % R], g == 0 ? p0c[vi / NOB] : p1[vi / NOB]);
        if (g == 1 && vi + R < NF) vf[vi % R] = P::v_frag(v_cur, vbase, vi + R);
        __builtin_amdgcn_sched_barrier(0);
      }
      exp_end(s0, 0, acc);
    }
    if constexpr (SUB == 1) {
      if constexpr (odd) {
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this pair of iterations' tile loads have landed
        lds_barrier();
      }
    } else {
      __builtin_amdgcn_s_waitcnt(0x0F70 | L::DMA_PER_WAVE);  // the previous iteration's tile has landed
      lds_barrier();
    }
  };

  // one pass over the keys; a second runs only if the first marked a row bad (see PassSoftmax)
  for (int pass = 0;; ++pass) {
#pragma unroll
    for (int g = 0; g < 2; ++g)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[g][db] = f32x16{};
    dma(k_tile(0), kb(0));
    dma(v_tile(0), vb(0));
    dma(k_tile(1), kb(1));
    if constexpr (SUB == 1) {  // the first pair of iterations reads K_1, K_2, V_0 and V_1
      dma(k_tile(2), kb(2));
      dma(v_tile(1), vb(1));
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this wave's tile loads have landed in LDS
    __syncthreads();
    // S_0 = K_0 Q^T, one K fragment per two MFMAs
#pragma unroll
    for (int kk = 0; kk < P::NQ; ++kk) {
      const bf16x8 kf = P::k_frag(kb(0), kbase, 2 * kk);
      if (kk == 0) {
        mfma_vgpr_first(s0, kf, qf[0].v[0]);
        mfma_vgpr_first(s1a, kf, qf[1].v[0]);
      } else {
        mfma_vgpr_acc(s0, kf, qf[0].v[kk]);
        mfma_vgpr_acc(s1a, kf, qf[1].v[kk]);
      }
    }
    s_result_guard<24>(s0, s1a);  // XDL result -> VALU read (row max below)
    __syncthreads();          // every wave is done with K_0 before its buffer is refilled
    if (nv_of(0) < kBNW) mask_scores(s0, s1a, nv_of(0));
    // the first tile's max is the reference of a first pass; group 0's exponentials are
    // taken here, group 1's (still in s1a) in the first iteration
    if (sm.m[0] == -__builtin_inff()) {
      sm.m[0] = row_max32(s0, c);
      sm.m[1] = row_max32(s1a, c);
    }
    {
      float xe[16], pe[16], acc = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) exp_slot(s0, 0, r, p0a, xe, pe, acc, 2);
      exp_end(s0, 0, acc);
    }
    // iterations 0 .. T2 - 1 with T2 = T rounded up to even: iteration j adds PV_j and takes
    // the scores of tile j + 1, so the last one or two iterations take phantom tiles at or past
    // T, whose keys are all masked (p = 0; their DMA zero-fills LDS without reading memory).
    // The PV product of tile T - 1 then needs no code of its own, and the loop body is one
    // pair of iterations, whose register sets alternate without copies.
    const int T2 = (T + 1) & ~1;
    for (int j = 0; j < T2; j += 2) {
      iteration(j, std::false_type{}, s1a, s1b, p0a, p0b);
      iteration(j + 1, std::true_type{}, s1b, s1a, p0b, p0a);
    }
    __builtin_amdgcn_s_waitcnt(0x0F70);  // no tile load may still be writing LDS when the pass ends
    if (!workgroup_redo(bad_flag, sm.bad, wave, lane) || pass > 0) break;
    sm.next_pass();
  }

  // the output rows are recomputed here rather than kept in registers through the loop
  int tid_e = threadIdx.x;
  asm volatile("" : "+v"(tid_e));
  Work we[2];
  we[0] = decode<PARTIAL>(a, kBMW, (tid_e >> 6) * 64 + (tid_e & 31));
  we[1] = next_group(a, we[0]);
  // every wave is past the barriers that end the pass, so the tile buffers are free: the
  // output rows of group g of wave w are staged in region 2 w + g
  static_assert(8 * 32 * D * 2 <= L::FLAGS, "eight groups' output rows fit the tile buffers");
#pragma unroll
  for (int g = 0; g < 2; ++g) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o_result_guard(o[g][db]);  // the epilogue reads O
    const float l = pair_sum(sm.l[g]);
    const float lse_nat = (sm.m[g] + __builtin_amdgcn_logf(l)) * kLn2;
    if constexpr (PARTIAL)
      write_rows<P, D, PARTIAL>(a, we[g], o[g], 1.0f / l, lse_nat, (tid_e >> 5) & 1);
    else
      write_out_staged<D>(a, we[g], o[g], 1.0f / l, lse_nat, (tid_e >> 5) & 1,
                          smem + (2 * (tid_e >> 6) + g) * (32 * D * 2), tid_e & 63);
  }
}

// ------------------------------------------------------------ LSE combine
// Merge of the C partials of one output row, four columns per thread: with
// M = max_c L_c, w_c = 2^((L_c - M) log2 e), out = sum_c w_c O_c / sum_c w_c and
// lse = M + ln sum_c w_c; M = -inf gives out = 0, lse = -inf.  pl points at L_0
// of the row (stride Tq between chunks), po at O_0 of the thread's columns
// (stride Tq * D).  Shared by the combine kernel and the single-launch split path
// so that both produce the same bits.
constexpr int kMergeRegs = 32;  // chunk counts up to this are merged from registers in one pass of loads

template <int D, bool OUT_F32>
__device__ __forceinline__ void merge_row4(const float* pl, const float* po, int C, int Tq, void* out, float* lse,
                                           int64_t row, int col) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  float mx = -__builtin_inff();
  if (C <= kMergeRegs) {
    // every chunk's statistic and partial in flight at once (one memory round trip per row);
    // the max, the weights and the sums are then taken in chunk order, as below
    float lc[kMergeRegs];
    f32x4 x[kMergeRegs];
#pragma unroll
    for (int u = 0; u < kMergeRegs; ++u) {
      lc[u] = -__builtin_inff();
      x[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u < C) {
        lc[u] = pl[(int64_t)u * Tq];
        x[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)u * Tq * D);
      }
    }
#pragma unroll
    for (int u = 0; u < kMergeRegs; ++u) mx = fmaxf(mx, lc[u]);
    if (mx != -__builtin_inff()) {
#pragma unroll
      for (int u = 0; u < kMergeRegs; ++u)
        if (u < C) {
          const float w = __builtin_amdgcn_exp2f((lc[u] - mx) * kLog2e);
          wsum += w;
          acc += w * x[u];
        }
      acc *= 1.0f / wsum;
    }
  } else {
    // eight chunks' loads in flight at a time; the sums still run in chunk order
    constexpr int U = 8;
    {
      int c = 0;
      for (; c + U <= C; c += U) {
        float lc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) lc[u] = pl[(int64_t)(c + u) * Tq];
#pragma unroll
        for (int u = 0; u < U; ++u) mx = fmaxf(mx, lc[u]);
      }
      for (; c < C; ++c) mx = fmaxf(mx, pl[(int64_t)c * Tq]);
    }
    if (mx != -__builtin_inff()) {
      int c = 0;
      for (; c + U <= C; c += U) {
        f32x4 x[U];
        float lc[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
          lc[u] = pl[(int64_t)(c + u) * Tq];
          x[u] = *reinterpret_cast<const f32x4*>(po + (int64_t)(c + u) * Tq * D);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
          const float w = __builtin_amdgcn_exp2f((lc[u] - mx) * kLog2e);
          wsum += w;
          acc += w * x[u];
        }
      }
      for (; c < C; ++c) {
        const float w = __builtin_amdgcn_exp2f((pl[(int64_t)c * Tq] - mx) * kLog2e);
        wsum += w;
        acc += w * *reinterpret_cast<const f32x4*>(po + (int64_t)c * Tq * D);
      }
      acc *= 1.0f / wsum;
    }
  }
  const int64_t off = row * D + col;
  if (OUT_F32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + off) = acc;
  } else {
    u32x2 w = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *reinterpret_cast<u32x2*>(reinterpret_cast<uint16_t*>(out) + off) = w;
  }
  if (lse && col == 0) lse[row] = (mx == -__builtin_inff()) ? mx : mx + __builtin_amdgcn_logf(wsum) * kLn2;
}

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
  const float* pl = a.part_lse + bh * a.C * a.Tq + i;              // stride Tq between chunks
  const float* po = a.part_out + (bh * a.C * a.Tq + i) * D + col;  // stride Tq*D between chunks
  merge_row4<D, OUT_F32>(pl, po, a.C, a.Tq, a.out, a.lse, row, col);
}

// Single-launch split-KV: after a chunk's workgroup has written its partial, it
// counts itself in for its (b, h, query tile); the workgroup that arrives last
// merges the C partials of that tile's rows (the same arithmetic as the combine
// kernel) and resets the count to zero for the next launch.  The eight XCDs
// have separate L2 caches, so the hand-off uses device-scope fences: a release
// (L2 write-back) before the count, an acquire (L2 invalidate) before the merge
// reads the other chunks' partials.
template <int D, bool OUT_F32>
__device__ __forceinline__ void splitkv_merge_tail(const FwdArgs& a) {
  __shared__ int s_last;
  int wg = blockIdx.x;
  const int qt = wg % a.n_qtiles;
  wg /= a.n_qtiles;
  wg /= a.C;
  const int h = wg % a.H, b = a.order_b ? longest_first(a.kv_len, a.B, a.S, wg / a.H) : wg / a.H;
  const int64_t bh = (int64_t)b * a.H + h;
  const int64_t cidx = bh * a.n_qtiles + qt;
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this thread's partial stores have reached L2
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");  // release at device scope (L2 write-back)
    s_last = (__hip_atomic_fetch_add(&a.counters[cidx], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == a.C - 1);
  }
  __syncthreads();
  if (!s_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // acquire (L2 invalidate): every chunk's partial is visible
  constexpr int TPR = D / 4, RPP = kThreads / TPR;  // threads per row, rows per pass
  const int col = (threadIdx.x % TPR) * 4;
  for (int r = threadIdx.x / TPR; r < kBM; r += RPP) {
    const int i = qt * kBM + r;
    if (i >= a.Tq) break;
    const float* pl = a.part_lse + bh * a.C * a.Tq + i;
    const float* po = a.part_out + (bh * a.C * a.Tq + i) * D + col;
    merge_row4<D, OUT_F32>(pl, po, a.C, a.Tq, a.out, a.lse, bh * a.Tq + i, col);
  }
  if (threadIdx.x == 0) a.counters[cidx] = 0;
}

// 64 query rows per wave at D = 256 and 128, bf16 (the host picks it, see plan_fwd).
template <int D, bool PARTIAL, bool STREAM>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void attn_fwd_wide_kernel(FwdArgs a) {
  __shared__ __attribute__((aligned(16))) char smem[WideLayout<D>::LDS_BYTES];
  bf16_fwd_wide<D, PARTIAL, STREAM>(a, smem);
}

// bf16 D = 256 launches split between the two paths in one grid: workgroups
// [0, n_wide) take the 64-row path over the rows that fill whole rounds of the GPU
// (wide.n_qtiles tiles of 256 per head), the rest the 32-row path over the remaining
// rows (narrow.row_base ..).  The workgroups of a launch then fill the machine more
// evenly than either kernel alone (e.g. 2 + 1 rounds instead of 2.5 or 5).
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(1, 1)))
void attn_fwd_mixed_kernel(FwdArgs wide, FwdArgs narrow, int n_wide) {
  constexpr int kBytes = WideLayout<256>::LDS_BYTES > dma_kernel_lds_bytes<256, 4>() ? WideLayout<256>::LDS_BYTES
                                                                                      : dma_kernel_lds_bytes<256, 4>();
  __shared__ __attribute__((aligned(16))) char smem[kBytes];  // one allocation serves both paths
  if ((int)blockIdx.x < n_wide) bf16_fwd_wide<256, false, false>(wide, smem);
  else bf16_fwd_dma<256, false, false>(narrow, smem);
}

// NW waves per workgroup (8 only for the bf16 fused forward at D <= 128, see bf16_fwd_dma).
template <class P, int D, bool PARTIAL, int WAVES_PER_EU, bool STREAM, bool MERGE = false, int NW = 4>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(WAVES_PER_EU, WAVES_PER_EU)))
void attn_fwd_kernel(FwdArgs a) {
  static_assert(!MERGE || PARTIAL, "the merge tail follows a partial");
  static_assert(NW == 4 || !P::kIsF32, "eight waves on the bf16 path only");
  if constexpr (P::kIsF32) {
    __shared__ __attribute__((aligned(16))) char smem[P::LDS_BYTES];
    attn_fwd_body<P, D, PARTIAL>(a, smem);
  } else {
    __shared__ __attribute__((aligned(16))) char smem[dma_kernel_lds_bytes<D, NW>()];
    bf16_fwd_dma<D, PARTIAL, STREAM, NW>(a, smem);
  }
  if constexpr (MERGE) splitkv_merge_tail<D, P::kIsF32>(a);
}

// ------------------------------------------------------- prefix mask -> kv_len
// One workgroup per batch row of a boolean key mask (one byte per key, nonzero =
// attend).  The row is a prefix mask exactly when its last nonzero byte comes
// before its first zero byte; then n_b = index of the first zero (S if none),
// otherwise -1.  This is the detection the page on tabfm PR #80 (section Fix)
// performs before rewriting a mask into a truncation, done on the device so the
// attention launch needs no host round trip for the lengths.  The row body is
// read as aligned 16-byte vectors; the unaligned head and the tail (under 16
// bytes each) are read bytewise by the first 32 lanes.
constexpr int kMaskThreads = 512;

// bit i set <=> byte i of w is nonzero (the carry of (b & 0x7f) + 0x7f stays in the byte)
__device__ __forceinline__ unsigned nonzero_bytes4(unsigned w) {
  const unsigned t = (((w & 0x7f7f7f7fu) + 0x7f7f7f7fu) | w) & 0x80808080u;
  return ((t >> 7) & 1u) | ((t >> 14) & 2u) | ((t >> 21) & 4u) | ((t >> 28) & 8u);
}

__global__ __launch_bounds__(kMaskThreads)
void prefix_mask_kernel(const uint8_t* mask, int S, int64_t row_stride, int32_t* kv_len) {
  const uint8_t* row = mask + (int64_t)blockIdx.x * row_stride;
  const int t = threadIdx.x;
  int first_zero = S, last_one = -1;
  const int mis = (int)(reinterpret_cast<uintptr_t>(row) & 15);
  const int head = min(S, (16 - mis) & 15);
  const int nvec = (S - head) >> 4;
  const int tail0 = head + (nvec << 4);
  if (t < 32) {
    const int j = t < 16 ? t : tail0 + (t - 16);
    if (j < (t < 16 ? head : S)) {
      if (row[j]) last_one = j;
      else first_zero = j;
    }
  }
  const uint4* vec = reinterpret_cast<const uint4*>(row + head);
  for (int i = t; i < nvec; i += kMaskThreads) {
    const uint4 w = vec[i];
    const unsigned nz = nonzero_bytes4(w.x) | (nonzero_bytes4(w.y) << 4) | (nonzero_bytes4(w.z) << 8) |
                        (nonzero_bytes4(w.w) << 12);
    const int o = head + (i << 4);
    if (nz) last_one = max(last_one, o + 31 - (int)__clz(nz));
    const unsigned z = ~nz & 0xffffu;
    if (z) first_zero = min(first_zero, o + __ffs(z) - 1);
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    first_zero = min(first_zero, __shfl_xor(first_zero, off));
    last_one = max(last_one, __shfl_xor(last_one, off));
  }
  constexpr int kWaves = kMaskThreads / 64;
  __shared__ int fz[kWaves], lo[kWaves];
  if ((t & 63) == 0) {
    fz[t >> 6] = first_zero;
    lo[t >> 6] = last_one;
  }
  __syncthreads();
  if (t == 0) {
    int f = fz[0], l = lo[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w) {
      f = min(f, fz[w]);
      l = max(l, lo[w]);
    }
    kv_len[blockIdx.x] = (l < f) ? f : -1;
  }
}

}  // namespace lcp
