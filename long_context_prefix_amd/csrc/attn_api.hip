// C ABI of libattnprefix.so: host-side validation, template choice and launch.
// Every argument check runs before the first HIP call, so a bad call returns
// its status code without touching the device.

#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "attn_bwd_kernels.hpp"
#include "attn_kernels.hpp"
#include "attn_prefix.h"

using namespace lcp;

namespace {

constexpr int64_t kMaxI32 = 2147483647;
// A 1-D dispatch counts work-items (workgroups x threads) in 32 bits, so a launch of wgs
// workgroups of `threads` threads fits only while wgs * threads < 2^32.
constexpr int64_t kMaxWorkItems = 4294967295LL;
bool grid_fits(int64_t wgs, int threads) { return wgs >= 0 && wgs <= kMaxWorkItems / threads; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Lazily filled caches below are atomics: calls from several host threads may fill them
// at once, each with the same value.
bool verbose() {
  static std::atomic<int> v{-1};
  int x = v.load(std::memory_order_relaxed);
  if (x < 0) {
    const char* e = getenv("ATTN_PREFIX_VERBOSE");
    x = (e && e[0] && e[0] != '0') ? 1 : 0;
    v.store(x, std::memory_order_relaxed);
  }
  return x == 1;
}

int esize(attn_dtype_t dt) { return dt == ATTN_F32 ? 4 : 2; }

// Checks shared by the fused and the split-KV forward.  On success *noop tells
// whether the call has no work at all (B, H or Tq is zero).
attn_status_t check_fwd(const void* q, const void* k, const void* v, const int32_t* kv_len, int B, int H,
                        int Tq, int S, int D, float scale, attn_dtype_t dtype, const void* out,
                        const void* out2, bool out2_required, int chunk_or_zero, bool split, bool* noop) {
  *noop = false;
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (B < 0 || H < 0 || Tq < 0 || S < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (split && (chunk_or_zero <= 0 || chunk_or_zero % kBN != 0)) return ATTN_ERR_CHUNK;
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  if (B == 0 || H == 0 || Tq == 0) {
    *noop = true;
    return ATTN_OK;
  }
  // sizes before pointers
  if ((int64_t)S * D * esize(dtype) > kMaxI32) return ATTN_ERR_SHAPE;
  const int64_t nqt = ((int64_t)Tq + kBM - 1) / kBM;
  int64_t grid = nqt * B * H;
  if (split) grid *= ((int64_t)S + chunk_or_zero - 1) / chunk_or_zero;
  if (!grid_fits(grid, kThreads)) return ATTN_ERR_SHAPE;
  if (!q || !kv_len || !out || (out2_required && !out2)) return ATTN_ERR_NULLPTR;
  if (S > 0 && (!k || !v)) return ATTN_ERR_NULLPTR;
  if (!aligned16(q) || !aligned16(out) || (out2 && !aligned4(out2)) || !aligned4(kv_len)) return ATTN_ERR_ALIGN;
  if (S > 0 && (!aligned16(k) || !aligned16(v))) return ATTN_ERR_ALIGN;
  return ATTN_OK;
}

template <class P, int D, bool PARTIAL, int W, bool MERGE>
attn_status_t launch_fwd(const FwdArgs& a, int64_t grid, hipStream_t stream, const char* tag) {
  // one query tile per head: every K/V tile is read by one workgroup, so stream it
  const bool stream_kv = !P::kIsF32 && a.n_qtiles == 1;
  if (verbose())
    fprintf(stderr, "[attn_prefix] %s D=%d %s grid=%lld block=%d lds=%d waves_per_eu=%d%s\n", tag, D,
            P::kIsF32 ? "f32" : "bf16", (long long)grid, kThreads, P::kIsF32 ? P::LDS_BYTES : dma_kernel_lds_bytes<D, 4>(),
            W, stream_kv ? " streaming" : "");
  (void)hipGetLastError();  // clear an error left by unrelated earlier calls
  if constexpr (!P::kIsF32) {
    if (stream_kv) {
      hipLaunchKernelGGL((attn_fwd_kernel<P, D, PARTIAL, W, true, MERGE>), dim3((unsigned)grid), dim3(kThreads), 0,
                         stream, a);
      return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
    }
  }
  hipLaunchKernelGGL((attn_fwd_kernel<P, D, PARTIAL, W, false, MERGE>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, a);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

template <bool PARTIAL, bool MERGE = false>
attn_status_t dispatch_fwd(const FwdArgs& a, int D, attn_dtype_t dtype, int64_t grid, hipStream_t s) {
  const char* tag = MERGE ? "splitkv_fwd" : (PARTIAL ? "splitkv_partial" : "prefix_fwd");
  if (dtype == ATTN_BF16) {
    switch (D) {
      case 64: return launch_fwd<Bf16Dma<64>, 64, PARTIAL, 2, MERGE>(a, grid, s, tag);
      case 128: return launch_fwd<Bf16Dma<128>, 128, PARTIAL, 2, MERGE>(a, grid, s, tag);
      case 256: return launch_fwd<Bf16Dma<256>, 256, PARTIAL, 1, MERGE>(a, grid, s, tag);
    }
  } else {
    switch (D) {
      case 64: return launch_fwd<F32Path<64>, 64, PARTIAL, 1, MERGE>(a, grid, s, tag);
      case 128: return launch_fwd<F32Path<128>, 128, PARTIAL, 1, MERGE>(a, grid, s, tag);
      case 256: return launch_fwd<F32Path<256>, 256, PARTIAL, 1, MERGE>(a, grid, s, tag);
    }
  }
  return ATTN_ERR_UNSUPPORTED;
}

// D = 256 or 128, bf16, 64 query rows per wave (256 per workgroup); plan_fwd decides when.
template <int D, bool PARTIAL>
attn_status_t launch_fwd_wide(FwdArgs a, int B, int H, hipStream_t stream, const char* tag) {
  a.n_qtiles = (a.Tq + kBMW - 1) / kBMW;
  const int64_t grid = (int64_t)a.n_qtiles * B * H * (PARTIAL ? a.C : 1);
  const bool stream_kv = a.n_qtiles == 1;
  if (verbose())
    fprintf(stderr, "[attn_prefix] %s D=%d bf16 wide grid=%lld block=%d lds=%d%s\n", tag, D, (long long)grid, kThreads,
            WideLayout<D>::LDS_BYTES, stream_kv ? " streaming" : "");
  (void)hipGetLastError();
  if (stream_kv)
    hipLaunchKernelGGL((attn_fwd_wide_kernel<D, PARTIAL, true>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_wide_kernel<D, PARTIAL, false>), dim3((unsigned)grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// The 32-row kernel with eight waves (256 query rows) per workgroup; bf16, D = 128 or 64,
// fused forward.
template <int D>
attn_status_t launch_fwd_8waves(FwdArgs a, int B, int H, hipStream_t stream) {
  a.n_qtiles = (a.Tq + kBM8 - 1) / kBM8;
  const int64_t grid = (int64_t)a.n_qtiles * B * H;
  if (!grid_fits(grid, 8 * 64)) return ATTN_ERR_SHAPE;  // (check_fwd counted 256-thread workgroups)
  if (verbose())
    fprintf(stderr, "[attn_prefix] prefix_fwd D=%d bf16 8 waves grid=%lld block=%d lds=%d\n", D, (long long)grid,
            8 * 64, dma_kernel_lds_bytes<D, 8>());
  (void)hipGetLastError();
  hipLaunchKernelGGL((attn_fwd_kernel<Bf16Dma<D>, D, false, 2, false, false, 8>), dim3((unsigned)grid), dim3(8 * 64),
                     0, stream, a);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus() {
  static std::atomic<int> cached[64];  // zero-initialized: not yet queried
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// Which D = 256 bf16 forward path a launch takes: the 32-row kernel, the 64-row kernel,
// or both in one grid (the 64-row path for the rows that fill whole rounds of the GPU, the
// 32-row path for the rest).  The 64-row path does about 8% more work per unit time, but
// its workgroups are twice as tall, so a last, partly filled round of them costs more.
// Each choice is costed in rounds of workgroups over the device's CUs, a 64-row round
// counting 2 / 1.08 of a 32-row one, and the cheapest is taken (ties to the simpler).
// ATTN_PREFIX_FWD_ROWS=128, 256 or mixed forces a choice (mixed: every full 256-row tile
// on the 64-row path).  At D = 128 the 64-row kernel is as fast as the 32-row one, not
// faster (its MFMAs wait on the softmax VALU work, which at D = 128 is twice as dense per
// MFMA), so it runs only when ATTN_PREFIX_FWD_ROWS=256 forces it.
//
// At D = 128 and 64 the 32-row kernel also comes with eight waves per workgroup (256 rows,
// one workgroup per CU; its tiles are loaded once per 256 rows and it waits and meets at a
// barrier every other tile), with the same bits.  At D = 128 it measured 1.5-2 % faster
// at ragged_32k and is taken when its workgroups fill at least one round of the CUs and
// need no more rounds than the four-wave ones (two per CU); at D = 64 it measured 0.4 %
// slower and runs only when forced.  ATTN_PREFIX_FWD_ROWS=128x8 forces it, =128 the
// four-wave form.
struct FwdPlan {
  int kind;        // 0: 32-row kernel, 1: 64-row kernel, 2: mixed, 3: 32-row kernel, 8 waves
  int wide_tiles;  // mixed: 256-row tiles per head on the 64-row path
};

FwdPlan plan_fwd(int D, attn_dtype_t dtype, int B, int H, int Tq) {
  FwdPlan p{0, 0};
  if (dtype != ATTN_BF16) return p;
  const char* e = getenv("ATTN_PREFIX_FWD_ROWS");
  const int64_t heads = (int64_t)B * H;
  if (D <= 128) {
    if (e && strcmp(e, "128") == 0) return p;
    if (e && strcmp(e, "128x8") == 0) return FwdPlan{3, 0};
    if (D == 128 && e && strcmp(e, "256") == 0) return FwdPlan{1, 0};
    if (D == 64) return p;
    const int64_t cus = device_cus();
    const int64_t wg8 = heads * ((Tq + kBM8 - 1) / kBM8), wg4 = heads * ((Tq + kBM - 1) / kBM);
    const bool fills = wg8 >= cus && (wg8 + cus - 1) / cus <= (wg4 + 2 * cus - 1) / (2 * cus);
    return fills ? FwdPlan{3, 0} : p;
  }
  const int64_t full_w = Tq / kBMW;  // full 256-row tiles per head
  if (e && strcmp(e, "128") == 0) return p;
  if (e && strcmp(e, "256") == 0) return FwdPlan{1, 0};
  if (e && strcmp(e, "mixed") == 0) {
    if (full_w == 0) return p;
    if (full_w * kBMW == Tq) return FwdPlan{1, 0};
    return FwdPlan{2, (int)full_w};
  }
  if (Tq <= kBM) return p;
  const int64_t cus = device_cus();
  auto rounds = [&](int64_t wgs) { return (wgs + cus - 1) / cus; };
  // costs in hundredths of a 32-row round
  const int64_t c_narrow = rounds(heads * ((Tq + kBM - 1) / kBM)) * 108;
  const int64_t c_wide = rounds(heads * ((Tq + kBMW - 1) / kBMW)) * 200;
  FwdPlan best = c_wide < c_narrow ? FwdPlan{1, 0} : p;
  int64_t c_best = c_wide < c_narrow ? c_wide : c_narrow;
  const int64_t w_rounds = heads * full_w / cus;  // whole rounds of full 256-row tiles
  if (w_rounds >= 1) {
    const int64_t W = (w_rounds * cus) / heads < full_w ? (w_rounds * cus) / heads : full_w;
    const int64_t rest = Tq - W * kBMW;
    if (W >= 1 && rest > 0) {
      const int64_t c_mixed = rounds(heads * W) * 200 + rounds(heads * ((rest + kBM - 1) / kBM)) * 108;
      if (c_mixed < c_best) best = FwdPlan{2, (int)W};
    }
  }
  return best;
}

// Both paths in one grid: the 64-row one over rows [0, 256 W) of every head, the 32-row
// one over the rest.
attn_status_t launch_fwd_mixed(const FwdArgs& base, int B, int H, int W, hipStream_t stream) {
  FwdArgs wide = base, narrow = base;
  wide.n_qtiles = W;
  narrow.row_base = W * kBMW;
  narrow.n_qtiles = (base.Tq - narrow.row_base + kBM - 1) / kBM;
  const int64_t n_wide = (int64_t)W * B * H;
  narrow.wg_base = (int)n_wide;
  const int64_t grid = n_wide + (int64_t)narrow.n_qtiles * B * H;
  if (verbose())
    fprintf(stderr, "[attn_prefix] prefix_fwd D=256 bf16 mixed grid=%lld (64-row %lld, 32-row %lld) lds=%d\n",
            (long long)grid, (long long)n_wide, (long long)(grid - n_wide), dma_kernel_lds_bytes<256, 4>());
  (void)hipGetLastError();
  hipLaunchKernelGGL(attn_fwd_mixed_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, wide, narrow,
                     (int)n_wide);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

// WPE_DKDV = 0 selects the cross-tile pipelined dk/dv kernel (one wave per SIMD), otherwise
// the slotted one at WPE_DKDV waves per SIMD.
template <int D, int WPE_DQ, int WPE_DKDV>
attn_status_t launch_bwd(const BwdArgs& base, int64_t rows, int64_t grid_dq, int64_t grid_dkdv, hipStream_t s) {
  (void)hipGetLastError();
  BwdArgs a = base;
  if (rows > 0) {
    constexpr int rows_per_wg = 256 / (D / 8);
    const int64_t g = (rows + rows_per_wg - 1) / rows_per_wg;
    hipLaunchKernelGGL((bwd_delta_kernel<D>), dim3((unsigned)g), dim3(256), 0, s, a, rows);
    a.n_tiles = (a.Tq + kBM - 1) / kBM;
    hipLaunchKernelGGL((bwd_dq_slot_kernel<D, WPE_DQ>), dim3((unsigned)grid_dq), dim3(kThreads), 0, s, a);
  }
  if (grid_dkdv > 0) {
    a.n_tiles = (a.S + 127) / 128;
    if constexpr (WPE_DKDV == 0)
      hipLaunchKernelGGL((bwd_dkdv_pipe_kernel<D>), dim3((unsigned)grid_dkdv), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_slot_kernel<D, WPE_DKDV>), dim3((unsigned)grid_dkdv), dim3(kThreads), 0, s, a);
  }
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // namespace

// Scratch of the allocation-free backward (attn_prefix_bwd_noalloc): its delta rows,
// rowsum(dout * out) in fp32, at most kNoAllocMaxRows of them.  A device array of the
// library's code object: every GPU the library runs on holds its own copy from the load
// of the library to the end of the process.  In host code `scratch` only names the
// symbol; its device address comes from hipGetSymbolAddress, per device.
constexpr int64_t kNoAllocMaxRows = int64_t(1) << 22;  // 16 MiB of fp32 per GPU
static __device__ __align__(256) float scratch[kNoAllocMaxRows];

namespace {

constexpr int kMaxDevices = 64;

// The device address of `scratch` on the current device, looked up once per device (with
// that device current) and kept; NULL when the lookup fails.
float* noalloc_scratch() {
  static std::atomic<float*> cached[kMaxDevices];  // zero-initialized: not yet looked up
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  float* p = cached[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = cached[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* addr = nullptr;
    if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) return nullptr;
    p = static_cast<float*>(addr);
    cached[dev].store(p, std::memory_order_release);
  }
  return p;
}

// The backward, with `delta` from the caller or (noalloc) in the library's scratch array.
attn_status_t prefix_bwd(const void* q, const void* k, const void* v, const int32_t* kv_len, const void* out,
                         const void* dout, const float* lse, int B, int H, int Tq, int S, int D, float scale,
                         attn_dtype_t dtype, float* delta, void* dq, void* dk, void* dv, void* stream, bool noalloc) {
  if (dtype != ATTN_BF16 && dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (B < 0 || H < 0 || Tq < 0 || S < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (dtype != ATTN_BF16 || (D != 64 && D != 128 && D != 256)) return ATTN_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return ATTN_ERR_ARG;
  if (B == 0 || H == 0 || (Tq == 0 && S == 0)) return ATTN_OK;
  // sizes before pointers
  if ((int64_t)S * D * 2 > kMaxI32) return ATTN_ERR_SHAPE;
  const int64_t rows = (int64_t)B * H * Tq;
  const int64_t grid_dq = (int64_t)B * H * ((Tq + kBM - 1) / kBM);
  const int64_t grid_dkdv = (int64_t)B * H * (((int64_t)S + 127) / 128);
  const int64_t grid_delta = (rows + 256 / (D / 8) - 1) / (256 / (D / 8));
  if (!grid_fits(grid_dq, kThreads) || !grid_fits(grid_dkdv, kThreads) || !grid_fits(grid_delta, 256))
    return ATTN_ERR_SHAPE;
  if (noalloc && rows > kNoAllocMaxRows) return ATTN_ERR_SHAPE;
  if (!kv_len) return ATTN_ERR_NULLPTR;
  if (Tq > 0 && (!q || !out || !dout || !lse || (!noalloc && !delta) || !dq)) return ATTN_ERR_NULLPTR;
  if (S > 0 && (!dk || !dv)) return ATTN_ERR_NULLPTR;
  if (S > 0 && Tq > 0 && (!k || !v)) return ATTN_ERR_NULLPTR;
  if (!aligned4(kv_len)) return ATTN_ERR_ALIGN;
  if (Tq > 0 && (!aligned16(q) || !aligned16(out) || !aligned16(dout) || !aligned16(dq) || !aligned4(lse) ||
                 (!noalloc && !aligned4(delta))))
    return ATTN_ERR_ALIGN;
  if (S > 0 && (!aligned16(dk) || !aligned16(dv) || (Tq > 0 && (!aligned16(k) || !aligned16(v)))))
    return ATTN_ERR_ALIGN;
  if (noalloc) {
    delta = noalloc_scratch();  // the first call on a device looks the address up
    if (!delta) return ATTN_ERR_HIP;
  }
  BwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_len = kv_len;
  a.out = out;
  a.dout = dout;
  a.lse = lse;
  a.delta = delta;
  a.B = B;
  a.H = H;
  a.Tq = Tq;
  a.S = S;
  a.scale = scale;
  a.scale_log2 = scale * kLog2e;
  a.order_b = (B > 1 && B <= kMaxOrderedBatch) ? 1 : 0;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  if (verbose())
    fprintf(stderr, "[attn_prefix] prefix_bwd%s D=%d B=%d H=%d Tq=%d S=%d grid dq=%lld dkdv=%lld\n",
            noalloc ? "_noalloc" : "", D, B, H, Tq, S, (long long)grid_dq, (long long)grid_dkdv);
  if (D == 64) return launch_bwd<64, 2, 2>(a, rows, grid_dq, grid_dkdv, st);
  if (D == 128) return launch_bwd<128, 2, 0>(a, rows, grid_dq, grid_dkdv, st);
  return launch_bwd<256, 1, 1>(a, rows, grid_dq, grid_dkdv, st);
}

}  // namespace

extern "C" {

int attn_version(void) { return (0 << 16) | (2 << 8) | 0; }

attn_status_t attn_prefix_mask_to_kv_len(const uint8_t* mask, int B, int S, int64_t row_stride, int32_t* kv_len,
                                         void* stream) {
  if (B < 0 || S < 0 || row_stride < 0) return ATTN_ERR_SHAPE;
  if (B == 0) return ATTN_OK;
  if (!grid_fits(B, kMaskThreads)) return ATTN_ERR_SHAPE;
  if (!kv_len || (S > 0 && !mask)) return ATTN_ERR_NULLPTR;
  if (!aligned4(kv_len)) return ATTN_ERR_ALIGN;
  if (verbose()) fprintf(stderr, "[attn_prefix] prefix_mask_to_kv_len B=%d S=%d\n", B, S);
  (void)hipGetLastError();
  hipLaunchKernelGGL(prefix_mask_kernel, dim3((unsigned)B), dim3(kMaskThreads), 0,
                     reinterpret_cast<hipStream_t>(stream), mask, S, row_stride, kv_len);
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

attn_status_t attn_prefix_bwd(const void* q, const void* k, const void* v, const int32_t* kv_len, const void* out,
                              const void* dout, const float* lse, int B, int H, int Tq, int S, int D, float scale,
                              attn_dtype_t dtype, float* delta, void* dq, void* dk, void* dv, void* stream) {
  return prefix_bwd(q, k, v, kv_len, out, dout, lse, B, H, Tq, S, D, scale, dtype, delta, dq, dk, dv, stream, false);
}

attn_status_t attn_prefix_bwd_noalloc(const void* q, const void* k, const void* v, const int32_t* kv_len,
                                      const void* out, const void* dout, const float* lse, int B, int H, int Tq,
                                      int S, int D, float scale, attn_dtype_t dtype, void* dq, void* dk, void* dv,
                                      void* stream) {
  return prefix_bwd(q, k, v, kv_len, out, dout, lse, B, H, Tq, S, D, scale, dtype, nullptr, dq, dk, dv, stream, true);
}

int attn_splitkv_num_chunks(int S, int chunk) {
  if (chunk <= 0 || S < 0) return -1;
  return (int)(((int64_t)S + chunk - 1) / chunk);
}

const char* attn_status_string(attn_status_t s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_ERR_NULLPTR: return "a required pointer is NULL";
    case ATTN_ERR_SHAPE: return "a size is negative or exceeds the library limits";
    case ATTN_ERR_DTYPE: return "unknown dtype (expected ATTN_BF16 or ATTN_F32)";
    case ATTN_ERR_UNSUPPORTED:
      return "unsupported head dim or dtype for this call (D 64/128/256; the backward takes bf16 only)";
    case ATTN_ERR_ALIGN: return "a tensor pointer is misaligned (16 bytes required; 4 for kv_len and lse)";
    case ATTN_ERR_CHUNK: return "chunk must be a positive multiple of 64";
    case ATTN_ERR_HIP: return "the HIP runtime reported an error";
    case ATTN_ERR_ARG: return "a scalar argument is out of range";
  }
  return "unknown status";
}

attn_status_t attn_prefix_fwd(const void* q, const void* k, const void* v, const int32_t* kv_len, int B, int H,
                              int Tq, int S, int D, float scale, attn_dtype_t dtype, void* out, float* lse,
                              void* stream) {
  bool noop = false;
  attn_status_t st = check_fwd(q, k, v, kv_len, B, H, Tq, S, D, scale, dtype, out, lse, false, 0, false, &noop);
  if (st != ATTN_OK || noop) return st;
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_len = kv_len;
  a.B = B;
  a.H = H;
  a.Tq = Tq;
  a.S = S;
  a.scale_log2 = scale * kLog2e;
  a.chunk = 0;
  a.C = 1;
  a.n_qtiles = (Tq + kBM - 1) / kBM;
  a.order_b = (B > 1 && B <= kMaxOrderedBatch) ? 1 : 0;
  a.out = out;
  a.lse = lse;
  const FwdPlan plan = plan_fwd(D, dtype, B, H, Tq);
  if (plan.kind == 1)
    return D == 128 ? launch_fwd_wide<128, false>(a, B, H, reinterpret_cast<hipStream_t>(stream), "prefix_fwd")
                    : launch_fwd_wide<256, false>(a, B, H, reinterpret_cast<hipStream_t>(stream), "prefix_fwd");
  if (plan.kind == 2) return launch_fwd_mixed(a, B, H, plan.wide_tiles, reinterpret_cast<hipStream_t>(stream));
  if (plan.kind == 3)
    return D == 128 ? launch_fwd_8waves<128>(a, B, H, reinterpret_cast<hipStream_t>(stream))
                    : launch_fwd_8waves<64>(a, B, H, reinterpret_cast<hipStream_t>(stream));
  const int64_t grid = (int64_t)a.n_qtiles * B * H;
  return dispatch_fwd<false>(a, D, dtype, grid, reinterpret_cast<hipStream_t>(stream));
}

attn_status_t attn_splitkv_partial(const void* q, const void* k, const void* v, const int32_t* kv_len, int B,
                                   int H, int Tq, int S, int D, float scale, attn_dtype_t dtype, int chunk,
                                   float* part_out, float* part_lse, void* stream) {
  bool noop = false;
  attn_status_t st =
      check_fwd(q, k, v, kv_len, B, H, Tq, S, D, scale, dtype, part_out, part_lse, true, chunk, true, &noop);
  if (st != ATTN_OK || noop) return st;
  const int C = attn_splitkv_num_chunks(S, chunk);
  if (C == 0) return ATTN_OK;  // S == 0: the partial tensors have no element
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_len = kv_len;
  a.B = B;
  a.H = H;
  a.Tq = Tq;
  a.S = S;
  a.scale_log2 = scale * kLog2e;
  a.chunk = chunk;
  a.C = C;
  a.n_qtiles = (Tq + kBM - 1) / kBM;
  a.order_b = (B > 1 && B <= kMaxOrderedBatch) ? 1 : 0;
  a.part_out = part_out;
  a.part_lse = part_lse;
  const int64_t grid = (int64_t)a.n_qtiles * C * B * H;
  return dispatch_fwd<true>(a, D, dtype, grid, reinterpret_cast<hipStream_t>(stream));
}

attn_status_t attn_splitkv_fwd(const void* q, const void* k, const void* v, const int32_t* kv_len, int B, int H,
                               int Tq, int S, int D, float scale, attn_dtype_t dtype, int chunk, float* part_out,
                               float* part_lse, int32_t* counters, void* out, float* lse, void* stream) {
  bool noop = false;
  attn_status_t st =
      check_fwd(q, k, v, kv_len, B, H, Tq, S, D, scale, dtype, part_out, part_lse, true, chunk, true, &noop);
  if (st != ATTN_OK || noop) return st;
  if (!counters || !out) return ATTN_ERR_NULLPTR;
  if (!aligned4(counters) || !aligned16(out) || (lse && !aligned4(lse))) return ATTN_ERR_ALIGN;
  const int C = attn_splitkv_num_chunks(S, chunk);
  if (C == 0) {  // S == 0: no key at all, so out = 0 and lse = -inf, which the combine writes for C = 0
    return attn_lse_combine(part_out, part_lse, B, H, 0, Tq, D, dtype, out, lse, stream);
  }
  FwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.kv_len = kv_len;
  a.B = B;
  a.H = H;
  a.Tq = Tq;
  a.S = S;
  a.scale_log2 = scale * kLog2e;
  a.chunk = chunk;
  a.C = C;
  a.n_qtiles = (Tq + kBM - 1) / kBM;
  a.order_b = (B > 1 && B <= kMaxOrderedBatch) ? 1 : 0;
  a.part_out = part_out;
  a.part_lse = part_lse;
  a.counters = counters;
  a.out = out;
  a.lse = lse;
  const int64_t grid = (int64_t)a.n_qtiles * C * B * H;
  return dispatch_fwd<true, true>(a, D, dtype, grid, reinterpret_cast<hipStream_t>(stream));
}

attn_status_t attn_lse_combine(const float* part_out, const float* part_lse, int B, int H, int C, int Tq, int D,
                               attn_dtype_t out_dtype, void* out, float* lse, void* stream) {
  if (out_dtype != ATTN_BF16 && out_dtype != ATTN_F32) return ATTN_ERR_DTYPE;
  if (B < 0 || H < 0 || C < 0 || Tq < 0 || D < 0) return ATTN_ERR_SHAPE;
  if (D != 64 && D != 128 && D != 256) return ATTN_ERR_UNSUPPORTED;
  if (B == 0 || H == 0 || Tq == 0) return ATTN_OK;
  const int64_t rows = (int64_t)B * H * Tq;
  const int rows_per_wg = 1024 / D;
  const int64_t grid = (rows + rows_per_wg - 1) / rows_per_wg;
  if (!grid_fits(grid, 256)) return ATTN_ERR_SHAPE;  // sizes before pointers
  if (!out || (C > 0 && (!part_out || !part_lse))) return ATTN_ERR_NULLPTR;
  if (!aligned16(out) || (lse && !aligned4(lse))) return ATTN_ERR_ALIGN;
  if (C > 0 && (!aligned16(part_out) || !aligned4(part_lse))) return ATTN_ERR_ALIGN;
  CombineArgs a{part_out, part_lse, rows, C, Tq, out, lse};
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (verbose())
    fprintf(stderr, "[attn_prefix] lse_combine D=%d C=%d %s grid=%lld\n", D, C, out_dtype == ATTN_F32 ? "f32" : "bf16",
            (long long)grid);
  (void)hipGetLastError();
#define LCP_COMBINE(DD, F32)                                                                                  \
  hipLaunchKernelGGL((lse_combine_kernel<DD, F32>), dim3((unsigned)grid), dim3(256), 0, s, a)
  if (out_dtype == ATTN_F32) {
    if (D == 64) LCP_COMBINE(64, true);
    else if (D == 128) LCP_COMBINE(128, true);
    else LCP_COMBINE(256, true);
  } else {
    if (D == 64) LCP_COMBINE(64, false);
    else if (D == 128) LCP_COMBINE(128, false);
    else LCP_COMBINE(256, false);
  }
#undef LCP_COMBINE
  return hipGetLastError() == hipSuccess ? ATTN_OK : ATTN_ERR_HIP;
}

}  // extern "C"
