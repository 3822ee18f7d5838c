// C ABI of the grouped block-scaled GEMM library (include/mxgg.h).
//
// Order inside every entry point: (1) argument validation (validate.hpp, no
// HIP calls), (2) the empty-batch return, (3) device checks -- the stream's
// GPU must be gfx950 (the scaled FP4/FP8 MFMA exists only on CDNA4, as the
// page "Triton mxfp4 (and a8w4) grouped GEMM kernel" states for its kernels)
// and every pointer must be device memory of that GPU (the operand's device,
// not merely the current one: "route te.GroupedLinear through #723; a8w4
// fwd-only") -- (4) kernel launches on the caller's stream. Nothing is enqueued
// before all checks pass.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstring>
#include <mutex>
#include <numeric>
#include <string>

#include "../../include/mxgg.h"
#include "launch.hpp"
#include "validate.hpp"

namespace mxgg {
namespace {

thread_local std::string g_last_error;

mxgg_status finish(const Check& c) {
  g_last_error = c.msg;
  return c.st;
}

mxgg_status ok() {
  g_last_error.clear();
  return MXGG_OK;
}

// Per-device cache: 0 unknown, 1 gfx950, 2 other arch.
constexpr int kMaxDevices = 64;
std::atomic<int> g_arch[kMaxDevices];
std::atomic<int> g_cus[kMaxDevices];

Check stream_device(hipStream_t st, int* dev) {
  hipError_t e = st ? hipStreamGetDevice(st, dev) : hipGetDevice(dev);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    Check r; r.st = MXGG_ERR_HIP; r.msg = std::string("cannot query the stream's device: ") + hipGetErrorString(e);
    return r;
  }
  if (*dev < 0 || *dev >= kMaxDevices) return fail(MXGG_ERR_DEVICE, "device ordinal %lld out of range", *dev);
  return Check{};
}

Check check_arch(int dev, int* num_cus) {
  int a = g_arch[dev].load(std::memory_order_acquire);
  if (a == 0) {
    hipDeviceProp_t prop;
    hipError_t e = hipGetDeviceProperties(&prop, dev);
    if (e != hipSuccess) {
      (void)hipGetLastError();
      Check r; r.st = MXGG_ERR_HIP; r.msg = std::string("hipGetDeviceProperties: ") + hipGetErrorString(e);
      return r;
    }
    a = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : 2;
    g_cus[dev].store(prop.multiProcessorCount, std::memory_order_relaxed);
    g_arch[dev].store(a, std::memory_order_release);
  }
  if (a != 1) return fail(MXGG_ERR_ARCH, "device %lld is not gfx950 (CDNA4 scaled MFMA required)", dev);
  *num_cus = g_cus[dev].load(std::memory_order_relaxed);
  return Check{};
}

Check check_on_device(const void* p, int dev, const char* name) {
  if (!p) return Check{};
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    Check r; r.st = MXGG_ERR_DEVICE; r.msg = std::string(name) + " is not HIP device memory";
    return r;
  }
  const bool devmem = attr.type == hipMemoryTypeDevice || attr.type == hipMemoryTypeManaged;
  if (!devmem || attr.device != dev) {
    Check r; r.st = MXGG_ERR_DEVICE;
    r.msg = std::string(name) + " is not device memory of the stream's GPU " + std::to_string(dev);
    return r;
  }
  return Check{};
}

// Arch + device membership of every pointer; returns the device's CU count.
Check device_checks(hipStream_t st, std::initializer_list<std::pair<const void*, const char*>> ptrs, int* num_cus) {
  int dev = 0;
  MXGG_TRY(stream_device(st, &dev));
  MXGG_TRY(check_arch(dev, num_cus));
  for (auto& pr : ptrs) MXGG_TRY(check_on_device(pr.first, dev, pr.second));
  return Check{};
}

Check hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return Check{};
  (void)hipGetLastError();
  Check r; r.st = MXGG_ERR_HIP; r.msg = std::string(what) + ": " + hipGetErrorString(e);
  return r;
}

SplitArgs make_splits(const int64_t* m, int32_t G) {
  SplitArgs s;
  std::memset(&s, 0, sizeof(s));
  s.G = G;
  for (int32_t g = 0; g < G; ++g) s.m[g] = (int32_t)m[g];
  return s;
}

}  // namespace
}  // namespace mxgg

using namespace mxgg;

extern "C" {

const char* mxgg_status_string(mxgg_status s) {
  switch (s) {
    case MXGG_OK: return "MXGG_OK";
    case MXGG_ERR_NULL: return "MXGG_ERR_NULL: a required pointer is NULL";
    case MXGG_ERR_SHAPE: return "MXGG_ERR_SHAPE: invalid expert count, dimension or leading dimension";
    case MXGG_ERR_SPLITS: return "MXGG_ERR_SPLITS: negative split or splits do not sum to the rows";
    case MXGG_ERR_FORMAT: return "MXGG_ERR_FORMAT: unsupported format or format pair";
    case MXGG_ERR_ALIGN: return "MXGG_ERR_ALIGN: misaligned pointer or leading dimension";
    case MXGG_ERR_WORKSPACE: return "MXGG_ERR_WORKSPACE: workspace too small";
    case MXGG_ERR_DEVICE: return "MXGG_ERR_DEVICE: pointer is not device memory of the stream's GPU";
    case MXGG_ERR_ARCH: return "MXGG_ERR_ARCH: the GPU is not gfx950";
    case MXGG_ERR_HIP: return "MXGG_ERR_HIP: HIP runtime or launch failure";
  }
  return "unknown mxgg_status";
}

const char* mxgg_last_error(void) { return g_last_error.c_str(); }

size_t mxgg_workspace_size(int32_t G) {
  (void)G;
  return 0;
}

int64_t mxgg_segpad_rows(const int64_t* m_splits, int32_t G, mxgg_format fmt) {
  if (!m_splits || G < 1 || G > MXGG_MAX_EXPERTS) return -1;
  fmt = (mxgg_format)base_format(format_bits(fmt));  // the scale layout does not change the padding
  if (fmt != MXGG_MXFP4 && fmt != MXGG_MXFP8 && fmt != MXGG_FP8_1x128) return -1;
  for (int32_t g = 0; g < G; ++g)
    if (m_splits[g] < 0 || m_splits[g] > kMaxSplit) return -1;
  return segpad_rows(m_splits, G, segpad_multiple(fmt));
}

int64_t mxgg_mx_scale_stride(int64_t rows) { return mx_scale_stride(rows); }

mxgg_status mxgg_mx_scales_relayout(const void* src, mxgg_scale_layout src_layout, int64_t rows, int64_t blocks,
                                    void* dst, mxgg_scale_layout dst_layout, hipStream_t stream) {
  Check c = validate_relayout(src, (int)src_layout, rows, blocks, dst, (int)dst_layout);
  if (!c.ok()) return finish(c);
  if (rows == 0) return ok();
  int cus = 0;
  c = device_checks(stream, {{src, "src"}, {dst, "dst"}}, &cus);
  if (!c.ok()) return finish(c);
  c = hip_status(launch_relayout_scales(static_cast<const uint8_t*>(src), (int)src_layout, rows, blocks,
                                        (int)dst_layout, static_cast<uint8_t*>(dst), stream),
                 "scale relayout launch");
  return c.ok() ? ok() : finish(c);
}

mxgg_status mxgg_quantize_rowwise(const void* x, int64_t rows, int64_t cols, int64_t ldx, mxgg_format fmt,
                                  uint32_t flags, void* q, void* scales, hipStream_t stream) {
  if (is_p2(fmt)) flags |= MXGG_POW2_SCALES;
  fmt = (mxgg_format)base_format(fmt);
  Check c = validate_quantize_rowwise(x, rows, cols, ldx, (int)fmt, q, scales);
  if (!c.ok()) return finish(c);
  if (rows == 0) return ok();
  const bool mfma = is_mfma_layout(fmt), kb = kblock_bits(fmt) != 0;
  fmt = (mxgg_format)format_bits(fmt);
  int cus = 0;
  c = device_checks(stream, {{x, "x"}, {q, "q"}, {scales, "scales"}}, &cus);
  if (!c.ok()) return finish(c);
  if (is_mx(fmt))
    c = hip_status(launch_quant_rowwise_mx(static_cast<const uint16_t*>(x), rows, cols, ldx, fmt == MXGG_MXFP8, mfma,
                                           kb, static_cast<uint8_t*>(q), static_cast<uint8_t*>(scales), cus, stream),
                   "row-wise quantizer launch");
  else
    c = hip_status(launch_quant_rowwise_blk(static_cast<const uint16_t*>(x), rows, cols, ldx,
                                            fmt == MXGG_FP8_128x128, (flags & MXGG_POW2_SCALES) != 0,
                                            static_cast<uint8_t*>(q), static_cast<float*>(scales), stream),
                   "blockwise quantizer launch");
  return c.ok() ? ok() : finish(c);
}

mxgg_status mxgg_quantize_colwise_segpad(const void* x, int64_t rows, int64_t cols, int64_t ldx,
                                         const int64_t* m_splits, int32_t G, mxgg_format fmt, uint32_t flags,
                                         void* q, void* scales, int64_t mpad, hipStream_t stream) {
  if (is_p2(fmt)) flags |= MXGG_POW2_SCALES;
  fmt = (mxgg_format)base_format(fmt);
  Check c = validate_quantize_colwise(x, rows, cols, ldx, m_splits, G, (int)fmt, q, scales, mpad);
  if (!c.ok()) return finish(c);
  if (rows == 0) return ok();
  const bool mfma = is_mfma_layout(fmt), kb = kblock_bits(fmt) != 0;
  fmt = (mxgg_format)format_bits(fmt);
  int cus = 0;
  c = device_checks(stream, {{x, "x"}, {q, "q"}, {scales, "scales"}}, &cus);
  if (!c.ok()) return finish(c);
  const SplitArgs sp = make_splits(m_splits, G);
  if (is_mx(fmt))
    c = hip_status(launch_quant_colwise_mx(static_cast<const uint16_t*>(x), rows, cols, ldx, sp, fmt == MXGG_MXFP8,
                                           mfma, kb, static_cast<uint8_t*>(q), static_cast<uint8_t*>(scales), mpad,
                                           cus, stream),
                   "column-wise quantizer launch");
  else
    c = hip_status(launch_quant_colwise_blk(static_cast<const uint16_t*>(x), cols, ldx, sp,
                                            (flags & MXGG_POW2_SCALES) != 0, static_cast<uint8_t*>(q),
                                            static_cast<float*>(scales), mpad, stream),
                   "blockwise column-wise quantizer launch");
  return c.ok() ? ok() : finish(c);
}

mxgg_status mxgg_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ldx, const int64_t* m_splits,
                               int32_t G, mxgg_format fmt, uint32_t flags, void* q_row, void* s_row, void* q_col,
                               void* s_col, int64_t mpad, hipStream_t stream) {
  if (is_p2(fmt)) flags |= MXGG_POW2_SCALES;
  fmt = (mxgg_format)base_format(fmt);
  Check c = validate_quantize_dual(x, rows, cols, ldx, m_splits, G, (int)fmt, q_row, s_row, q_col, s_col, mpad);
  if (!c.ok()) return finish(c);
  if (rows == 0) return ok();
  const bool mfma = is_mfma_layout(fmt);
  const bool kbr = (fmt & MXGG_KBLOCK_ROWS) != 0, kbc = (fmt & MXGG_KBLOCK_COLS) != 0;
  fmt = (mxgg_format)format_bits(fmt);
  int cus = 0;
  c = device_checks(stream, {{x, "x"}, {q_row, "q_row"}, {s_row, "s_row"}, {q_col, "q_col"}, {s_col, "s_col"}}, &cus);
  if (!c.ok()) return finish(c);
  const SplitArgs sp = make_splits(m_splits, G);
  if (is_mx(fmt))
    c = hip_status(launch_quant_dual_mx(static_cast<const uint16_t*>(x), rows, cols, ldx, sp, fmt == MXGG_MXFP8, mfma,
                                        kbr, kbc, static_cast<uint8_t*>(q_row), static_cast<uint8_t*>(s_row),
                                        static_cast<uint8_t*>(q_col), static_cast<uint8_t*>(s_col), mpad, cus,
                                        stream),
                   "dual quantizer launch");
  else
    c = hip_status(launch_quant_dual_blk(static_cast<const uint16_t*>(x), rows, cols, ldx, sp,
                                         (flags & MXGG_POW2_SCALES) != 0, static_cast<uint8_t*>(q_row),
                                         static_cast<float*>(s_row), static_cast<uint8_t*>(q_col),
                                         static_cast<float*>(s_col), mpad, stream),
                   "blockwise dual quantizer launch");
  return c.ok() ? ok() : finish(c);
}

mxgg_status mxgg_transpose_128x128(const void* w_q, const void* w_s, int32_t G, int64_t N, int64_t K, void* wt_q,
                                   void* wt_s, hipStream_t stream) {
  Check c = validate_transpose_128x128(w_q, w_s, G, N, K, wt_q, wt_s);
  if (!c.ok()) return finish(c);
  int cus = 0;
  c = device_checks(stream, {{w_q, "w_q"}, {w_s, "w_s"}, {wt_q, "wt_q"}, {wt_s, "wt_s"}}, &cus);
  if (!c.ok()) return finish(c);
  c = hip_status(launch_transpose_128x128(static_cast<const uint8_t*>(w_q), static_cast<const float*>(w_s), G, N, K,
                                          static_cast<uint8_t*>(wt_q), static_cast<float*>(wt_s), stream),
                 "transpose launch");
  return c.ok() ? ok() : finish(c);
}

mxgg_status mxgg_grouped_fwd(const void* a_q, const void* a_s, mxgg_format a_fmt, const void* w_q, const void* w_s,
                             mxgg_format w_fmt, const int64_t* m_splits, int32_t G, int64_t M, int64_t N, int64_t K,
                             void* out, void* ws, size_t ws_bytes, hipStream_t stream) {
  // power-of-two blockwise scales on both sides: the MFMA applies them
  const bool p2 = is_p2(a_fmt) && is_p2(w_fmt);
  a_fmt = (mxgg_format)base_format(a_fmt);
  w_fmt = (mxgg_format)base_format(w_fmt);
  Check c = validate_fwd(a_q, a_s, (int)a_fmt, w_q, w_s, (int)w_fmt, m_splits, G, M, N, K, out, ws, ws_bytes,
                         mxgg_workspace_size(G));
  if (!c.ok()) return finish(c);
  if (M == 0) return ok();
  const bool w_mfma = is_mfma_layout(w_fmt), kb = kblock_bits(a_fmt) != 0;
  a_fmt = (mxgg_format)format_bits(a_fmt);
  w_fmt = (mxgg_format)format_bits(w_fmt);
  int cus = 0;
  c = device_checks(stream, {{a_q, "a_q"}, {a_s, "a_s"}, {w_q, "w_q"}, {w_s, "w_s"}, {out, "out"}}, &cus);
  if (!c.ok()) return finish(c);
  RowsGemmParams p;
  std::memset(&p, 0, sizeof(p));
  if (a_fmt == MXGG_FP8_1x128) {
    // E4M3 x E4M3 in 64-byte K blocks (A [K/64, M, 64], W [K/64, G*N, 64]);
    // A scales f32 [K/128, M] (block-major), W scales f32 [G*N/128, K/128]
    p.a = static_cast<const uint8_t*>(a_q);
    p.as = static_cast<const uint8_t*>(a_s);
    p.b = static_cast<const uint8_t*>(w_q);
    p.bs = static_cast<const uint8_t*>(w_s);
    p.c = static_cast<uint16_t*>(out);
    p.lda = M * 64;  // bytes per K block
    p.ldas = M * 4;
    p.ldb = (int64_t)G * N * 64;
    p.ldbs = K / 128 * 4;
    p.b_gstride = N * 64;  // expert g's rows start at g*N in every K block
    p.bs_gstride = N / 128 * (K / 128 * 4);
    p.ldc = N;
    p.n_out = (int32_t)N;
    p.kc = (int32_t)K;
    p.sp = make_splits(m_splits, G);
    c = hip_status(launch_grouped_rows_blk(p, p2, false, cus, stream), "blockwise forward launch");
    return c.ok() ? ok() : finish(c);
  }
  const bool a8 = a_fmt == MXGG_MXFP8;
  p.a = static_cast<const uint8_t*>(a_q);
  p.as = static_cast<const uint8_t*>(a_s);
  p.b = static_cast<const uint8_t*>(w_q);
  p.bs = static_cast<const uint8_t*>(w_s);
  p.c = static_cast<uint16_t*>(out);
  // codes in rows, or in 64-byte K blocks (ld = bytes per block: rows * 64)
  p.lda = kb ? M * 64 : a8 ? K : K / 2;
  p.ldas = mx_scale_stride(M);    // A scales [K/32, R4(M)]
  p.ldb = kb ? (int64_t)G * N * 64 : K / 2;
  p.ldbs = (int64_t)G * N;        // W scales [K/32, G*N] (MFMA layout: a 128-element
                                  // group is 4 blocks of G*N bytes, N % 32 == 0)
  p.b_gstride = kb ? N * 64 : N * (K / 2);
  p.bs_gstride = w_mfma ? N * 4 : N;  // expert g's rows start at g*N (its units at byte g*N*4)
  p.ldc = N;
  p.n_out = (int32_t)N;
  p.kc = (int32_t)K;
  p.sp = make_splits(m_splits, G);
  c = hip_status(launch_grouped_rows_mx(p, a8, false, w_mfma, kb, cus, stream), "forward launch");
  return c.ok() ? ok() : finish(c);
}

mxgg_status mxgg_grouped_dgrad(const void* dy_q, const void* dy_s, const void* wcol_q, const void* wcol_s,
                               mxgg_format fmt, const int64_t* m_splits, int32_t G, int64_t M, int64_t N, int64_t K,
                               void* dx, void* ws, size_t ws_bytes, hipStream_t stream) {
  const bool p2 = is_p2(fmt);
  fmt = (mxgg_format)base_format(fmt);
  Check c = validate_dgrad(dy_q, dy_s, wcol_q, wcol_s, (int)fmt, m_splits, G, M, N, K, dx, ws, ws_bytes,
                           mxgg_workspace_size(G));
  if (!c.ok()) return finish(c);
  if (M == 0) return ok();
  const bool w_mfma = is_mfma_layout(fmt), kb = kblock_bits(fmt) != 0;
  fmt = (mxgg_format)format_bits(fmt);
  int cus = 0;
  c = device_checks(stream, {{dy_q, "dy_q"}, {dy_s, "dy_s"}, {wcol_q, "wcol_q"}, {wcol_s, "wcol_s"}, {dx, "dx"}},
                    &cus);
  if (!c.ok()) return finish(c);
  RowsGemmParams p;
  std::memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(dy_q);
  p.as = static_cast<const uint8_t*>(dy_s);
  p.b = static_cast<const uint8_t*>(wcol_q);
  p.bs = static_cast<const uint8_t*>(wcol_s);
  p.c = static_cast<uint16_t*>(dx);
  p.ldc = K;
  p.n_out = (int32_t)K;
  p.kc = (int32_t)N;
  p.sp = make_splits(m_splits, G);
  if (fmt == MXGG_FP8_1x128) {
    // dY E4M3 [N/64, M, 64] + f32 [N/128, M]; W^T E4M3 [N/64, G*K, 64] + f32
    // [G*K/128, N/128]
    // (the 128x128 blocks of W, transposed: same codes, same scales)
    p.lda = M * 64;
    p.ldas = M * 4;
    p.ldb = (int64_t)G * K * 64;
    p.ldbs = N / 128 * 4;
    p.b_gstride = K * 64;
    p.bs_gstride = K / 128 * (N / 128 * 4);
    c = hip_status(launch_grouped_rows_blk(p, p2, true, cus, stream), "blockwise dgrad launch");
    return c.ok() ? ok() : finish(c);
  }
  const bool a8 = fmt == MXGG_MXFP8;  // a8w4: dY E4M3, W E2M1
  // codes in rows, or in 64-byte K blocks (ld = bytes per block: rows * 64)
  p.lda = kb ? M * 64 : a8 ? N : N / 2;
  p.ldas = mx_scale_stride(M);    // dY scales [N/32, R4(M)]
  p.ldb = kb ? K * 64 : (int64_t)G * N / 2;  // W column-wise: [K, G*N/2] (blocked: [G*N/128, K, 64])
  p.ldbs = K;                     // its scales [G*N/32, K] (MFMA layout: 4 blocks of K
                                  // bytes per 128-element group)
  p.b_gstride = kb ? N / 128 * K * 64 : N / 2;  // expert g owns columns [g*N, (g+1)*N)
  p.bs_gstride = N / 32 * K;      // ... and scale blocks [g*N/32, (g+1)*N/32) (MFMA: the
                                  // same byte offset, groups [g*N/128, (g+1)*N/128))
  c = hip_status(launch_grouped_rows_mx(p, a8, true, w_mfma, kb, cus, stream), "dgrad launch");
  return c.ok() ? ok() : finish(c);
}

mxgg_status mxgg_grouped_wgrad(const void* dycol_q, const void* dycol_s, const void* xcol_q, const void* xcol_s,
                               mxgg_format fmt, const int64_t* m_splits, int32_t G, int64_t N, int64_t K,
                               int64_t mpad, void* main_grad, int32_t out_is_bf16, int32_t accumulate, void* ws,
                               size_t ws_bytes, hipStream_t stream) {
  const bool p2 = is_p2(fmt);
  fmt = (mxgg_format)base_format(fmt);
  Check c = validate_wgrad(dycol_q, dycol_s, xcol_q, xcol_s, (int)fmt, m_splits, G, N, K, mpad, main_grad,
                           out_is_bf16, accumulate, ws, ws_bytes, mxgg_workspace_size(G));
  if (!c.ok()) return finish(c);
  if (mpad == 0 && accumulate) return ok();
  const bool blk = fmt == MXGG_FP8_1x128;
  const bool fp8 = fmt == MXGG_MXFP8;
  int cus = 0;
  c = device_checks(stream, {{dycol_q, "dycol_q"}, {dycol_s, "dycol_s"}, {xcol_q, "xcol_q"}, {xcol_s, "xcol_s"},
                             {main_grad, "main_grad"}},
                    &cus);
  if (!c.ok()) return finish(c);
  WgradParams p;
  std::memset(&p, 0, sizeof(p));
  p.a = static_cast<const uint8_t*>(dycol_q);
  p.as = static_cast<const uint8_t*>(dycol_s);
  p.b = static_cast<const uint8_t*>(xcol_q);
  p.bs = static_cast<const uint8_t*>(xcol_s);
  p.c = main_grad;
  // row strides of the [N, mpad] / [K, mpad] codes (E4M3 / E2M1 bytes);
  // blockwise: bytes per 64-byte K block, u8 [mpad/64, N or K, 64]
  p.lda = blk ? N * 64 : fp8 ? mpad : mpad / 2;
  p.ldb = blk ? K * 64 : p.lda;
  p.ldas = blk ? N * 4 : N;                      // f32 [mpad/128, N] / u8 [mpad/32, N]
  p.ldbs = blk ? K * 4 : K;                      // f32 [mpad/128, K] / u8 [mpad/32, K]
  p.n_rows = (int32_t)N;
  p.n_cols = (int32_t)K;
  p.accumulate = accumulate;
  p.out_bf16 = out_is_bf16;
  p.sp = make_splits(m_splits, G);
  // longest expert first: the variable-K tiles of big experts start early
  int order[MXGG_MAX_EXPERTS];
  std::iota(order, order + G, 0);
  std::stable_sort(order, order + G, [&](int x, int y) { return m_splits[x] > m_splits[y]; });
  for (int32_t j = 0; j < G; ++j) p.order[j] = (int16_t)order[j];
  c = hip_status(blk ? launch_grouped_wgrad_blk(p, p2, cus, stream) : launch_grouped_wgrad_mx(p, fp8, cus, stream),
                 "wgrad launch");
  return c.ok() ? ok() : finish(c);
}

}  // extern "C"
