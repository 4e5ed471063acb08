// Exported device entry points of libssg: argument validation on the host,
// a cached per-device architecture check, then one kernel launch on the
// caller's stream.  Nothing is allocated and nothing is synchronised.
#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>

#include "kernels/launch.h"
#include "status.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other architecture
int g_arch_state[kMaxDevices] = {0};
std::mutex g_arch_mu;

// SSG_OK if a gfx950 device is current; SSG_ENODEV / SSG_EARCH / SSG_EHIP otherwise.
int check_device() {
    int count = 0;
    hipError_t e = hipGetDeviceCount(&count);
    if (e != hipSuccess || count <= 0) return ssg::fail(SSG_ENODEV, "no HIP device visible");
    int dev = 0;
    e = hipGetDevice(&dev);
    if (e != hipSuccess) return ssg::fail(SSG_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return ssg::fail(SSG_ENODEV, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_arch_mu);
    if (g_arch_state[dev] == 0) {
        hipDeviceProp_t prop;
        e = hipGetDeviceProperties(&prop, dev);
        if (e != hipSuccess) return ssg::fail(SSG_EHIP, "hipGetDeviceProperties: %s", hipGetErrorString(e));
        g_arch_state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
        if (g_arch_state[dev] == 2)
            return ssg::fail(SSG_EARCH, "device %d is %s, this library targets gfx950", dev, prop.gcnArchName);
    }
    if (g_arch_state[dev] != 1) return ssg::fail(SSG_EARCH, "device %d is not gfx950", dev);
    return SSG_OK;
}

int launched(hipError_t e, const char *what) {
    if (e != hipSuccess) return ssg::fail(SSG_EHIP, "%s launch failed: %s", what, hipGetErrorString(e));
    ssg::clear_error();
    return SSG_OK;
}

bool fits_int(int64_t v) { return v >= 0 && v < (int64_t(1) << 31); }

// Common shape / pointer checks for the row-major GEMMs.
int check_gemm(const char *fn, const void *A, const void *W, const void *C, int64_t M, int64_t N, int64_t K,
               int k_mult, int n_mult) {
    if (M < 0 || N <= 0 || K <= 0)
        return ssg::fail(SSG_EINVAL, "%s: M=%lld N=%lld K=%lld (need M >= 0, N > 0, K > 0)", fn, (long long)M,
                         (long long)N, (long long)K);
    if (!fits_int(M) || !fits_int(N) || !fits_int(K) || !fits_int(M / 64 * N / 64))
        return ssg::fail(SSG_EINVAL, "%s: dimensions too large", fn);
    if (K % k_mult) return ssg::fail(SSG_EINVAL, "%s: K=%lld must be a multiple of %d", fn, (long long)K, k_mult);
    if (N % n_mult) return ssg::fail(SSG_EINVAL, "%s: N=%lld must be a multiple of %d", fn, (long long)N, n_mult);
    if (M == 0) return SSG_OK;
    // the kernels address A and W with 32-bit byte offsets
    if (M * K * 2 >= (int64_t(1) << 32) || N * K * 2 >= (int64_t(1) << 32))
        return ssg::fail(SSG_EINVAL, "%s: A or W larger than 4 GiB", fn);
    if (!A || !W || !C) return ssg::fail(SSG_EINVAL, "%s: null pointer", fn);
    if (!ssg::aligned16(A) || !ssg::aligned16(W) || !ssg::aligned16(C))
        return ssg::fail(SSG_EINVAL, "%s: pointers must be 16-byte aligned", fn);
    return SSG_OK;
}

}  // namespace

SSG_API int ssg_device_arch(char *buf, int64_t len) {
    if (!buf || len <= 0) return ssg::fail(SSG_EINVAL, "ssg_device_arch: bad buffer");
    int count = 0;
    if (hipGetDeviceCount(&count) != hipSuccess || count <= 0) return ssg::fail(SSG_ENODEV, "no HIP device visible");
    int dev = 0;
    hipDeviceProp_t prop;
    if (hipGetDevice(&dev) != hipSuccess || hipGetDeviceProperties(&prop, dev) != hipSuccess)
        return ssg::fail(SSG_EHIP, "cannot query the current device");
    std::strncpy(buf, prop.gcnArchName, size_t(len) - 1);
    buf[len - 1] = '\0';
    ssg::clear_error();
    return SSG_OK;
}

SSG_API int dense_gemm_f16(const void *A, const void *Wt, void *C, int64_t M, int64_t N, int64_t K, void *stream) {
    int rc = check_gemm("dense_gemm_f16", A, Wt, C, M, N, K, 64, 64);
    if (rc || M == 0) return rc ? rc : (ssg::clear_error(), SSG_OK);
    if ((rc = check_device())) return rc;
    return launched(ssg::launch_dense_f16(A, Wt, C, int(M), int(N), int(K), hipStream_t(stream)), "dense_gemm_f16");
}

namespace {

// Checks shared by the int8 GEMMs' epilogue arguments.
int check_i8_epilogue(const char *fn, const float *scale, const float *bias, int out) {
    if (out < ssg::OUT_I32 || out > ssg::OUT_I8) return ssg::fail(SSG_EINVAL, "%s: unknown out_type %d", fn, out);
    if (out == ssg::OUT_I32 && (scale || bias))
        return ssg::fail(SSG_EINVAL, "%s: SSG_OUT_I32 takes no scale or bias", fn);
    if (out != ssg::OUT_I32 && !scale) return ssg::fail(SSG_EINVAL, "%s: this out_type needs scale", fn);
    if ((scale && !ssg::aligned16(scale)) || (bias && !ssg::aligned16(bias)))
        return ssg::fail(SSG_EINVAL, "%s: scale and bias must be 16-byte aligned", fn);
    return SSG_OK;
}

int dense_i8(const char *fn, const int8_t *A, const int8_t *Wt, const float *scale, const float *bias, void *C,
             int out, int64_t M, int64_t N, int64_t K, void *stream) {
    int rc = check_gemm(fn, A, Wt, C, M, N, K, 128, 64);
    if (rc || M == 0) return rc ? rc : (ssg::clear_error(), SSG_OK);
    if ((rc = check_i8_epilogue(fn, scale, bias, out))) return rc;
    if ((rc = check_device())) return rc;
    return launched(ssg::launch_dense_i8(A, Wt, scale, bias, C, out, int(M), int(N), int(K), hipStream_t(stream)), fn);
}

int w24_i8(const char *fn, const int8_t *A, const int8_t *vals, const uint32_t *meta, const float *scale,
           const float *bias, void *C, int out, int64_t M, int64_t N, int64_t K, void *stream) {
    int rc = check_gemm(fn, A, vals, C, M, N, K, 128, 64);
    if (rc || M == 0) return rc ? rc : (ssg::clear_error(), SSG_OK);
    if (!meta || !ssg::aligned16(meta)) return ssg::fail(SSG_EINVAL, "%s: meta null or misaligned", fn);
    if ((rc = check_i8_epilogue(fn, scale, bias, out))) return rc;
    if ((rc = check_device())) return rc;
    return launched(ssg::launch_w24_i8(A, vals, meta, scale, bias, C, out, int(M), int(N), int(K), hipStream_t(stream)),
                    fn);
}

}  // namespace

SSG_API int dense_gemm_i8(const int8_t *A, const int8_t *Wt, const float *scale, void *C, int64_t M, int64_t N,
                          int64_t K, void *stream) {
    return dense_i8("dense_gemm_i8", A, Wt, scale, nullptr, C, scale ? ssg::OUT_F32 : ssg::OUT_I32, M, N, K, stream);
}

SSG_API int dense_gemm_i8_out(const int8_t *A, const int8_t *Wt, const float *scale, const float *bias, void *C,
                              int32_t out_type, int64_t M, int64_t N, int64_t K, void *stream) {
    return dense_i8("dense_gemm_i8_out", A, Wt, scale, bias, C, out_type, M, N, K, stream);
}

SSG_API int w24_gemm_f16(const void *A, const void *vals, const uint32_t *meta, void *C, int64_t M, int64_t N,
                         int64_t K, void *stream) {
    int rc = check_gemm("w24_gemm_f16", A, vals, C, M, N, K, 64, 64);
    if (rc || M == 0) return rc ? rc : (ssg::clear_error(), SSG_OK);
    if (!meta || !ssg::aligned16(meta)) return ssg::fail(SSG_EINVAL, "w24_gemm_f16: meta null or misaligned");
    if ((rc = check_device())) return rc;
    return launched(ssg::launch_w24_f16(A, vals, meta, C, int(M), int(N), int(K), hipStream_t(stream)),
                    "w24_gemm_f16");
}

SSG_API int w24_gemm_i8(const int8_t *A, const int8_t *vals, const uint32_t *meta, const float *scale, void *C,
                        int64_t M, int64_t N, int64_t K, void *stream) {
    return w24_i8("w24_gemm_i8", A, vals, meta, scale, nullptr, C, scale ? ssg::OUT_F32 : ssg::OUT_I32, M, N, K,
                  stream);
}

SSG_API int w24_gemm_i8_out(const int8_t *A, const int8_t *vals, const uint32_t *meta, const float *scale,
                            const float *bias, void *C, int32_t out_type, int64_t M, int64_t N, int64_t K,
                            void *stream) {
    return w24_i8("w24_gemm_i8_out", A, vals, meta, scale, bias, C, out_type, M, N, K, stream);
}

namespace {

// Split K: check the split arguments, run the partial launch and the reduce
// launch on the caller's stream (kinds as in kernels/launch.h).
int split_run(const char *fn, int kind, const void *A, const void *W, const uint32_t *meta, const float *scale,
              const float *bias, void *C, int out, int64_t M, int64_t N, int64_t K, int32_t splits, void *ws,
              int64_t ws_bytes, void *stream) {
    const bool i8 = kind == 2 || kind == 3;
    int rc = check_gemm(fn, A, W, C, M, N, K, i8 ? 128 : 64, 64);
    if (rc) return rc;
    if (kind == 1 || kind == 3)
        if (M > 0 && (!meta || !ssg::aligned16(meta))) return ssg::fail(SSG_EINVAL, "%s: meta null or misaligned", fn);
    if (i8 && (rc = check_i8_epilogue(fn, scale, bias, out))) return rc;
    const int stages = ssg::gemm_k_stages(kind, int(K));
    if (splits < 1 || splits > 64 || stages % splits)
        return ssg::fail(SSG_EINVAL, "%s: splits=%d must be in 1..64 and divide the %d K stages", fn, int(splits),
                         stages);
    if (M == 0) return (ssg::clear_error(), SSG_OK);
    if (splits > 1) {
        if (!ws || !ssg::aligned16(ws)) return ssg::fail(SSG_EINVAL, "%s: workspace null or not 16-byte aligned", fn);
        const int64_t need = int64_t(splits) * M * N * 4;
        if (ws_bytes < need)
            return ssg::fail(SSG_EINVAL, "%s: workspace of %lld bytes, %lld needed", fn, (long long)ws_bytes,
                             (long long)need);
    }
    if ((rc = check_device())) return rc;
    const hipStream_t st = hipStream_t(stream);
    if (splits == 1) {
        switch (kind) {
            case 0: return launched(ssg::launch_dense_f16(A, W, C, int(M), int(N), int(K), st), fn);
            case 1: return launched(ssg::launch_w24_f16(A, W, meta, C, int(M), int(N), int(K), st), fn);
            case 2:
                return launched(ssg::launch_dense_i8(A, W, scale, bias, C, out, int(M), int(N), int(K), st), fn);
            default:
                return launched(ssg::launch_w24_i8(A, W, meta, scale, bias, C, out, int(M), int(N), int(K), st), fn);
        }
    }
    rc = launched(ssg::launch_gemm_partials(kind, A, W, meta, ws, int(M), int(N), int(K), int(splits), st), fn);
    if (rc) return rc;
    return launched(ssg::launch_splitk_reduce(ws, int(splits), i8, scale, bias, C, out, int(M), int(N), st), fn);
}

}  // namespace

SSG_API int64_t ssg_splitk_workspace_bytes(int64_t M, int64_t N, int32_t splits) {
    if (splits <= 1 || M <= 0 || N <= 0) return 0;
    return int64_t(splits) * M * N * 4;
}

SSG_API int32_t ssg_splitk_suggest(int32_t kind, int64_t M, int64_t N, int64_t K) {
    if (kind < 0 || kind > 3 || !fits_int(M) || !fits_int(N) || !fits_int(K)) return 1;
    return ssg::suggest_splits(int(kind), int(M), int(N), int(K));
}

SSG_API int32_t ssg_tile_choice(int32_t kind, int64_t M, int64_t N, int64_t K) {
    if (kind < 0 || kind > 3 || M <= 0 || N <= 0 || K <= 0 || !fits_int(M) || !fits_int(N) || !fits_int(K)) return 0;
    int bm = 0, bn = 0;
    ssg::tile_choice(int(kind), int(M), int(N), int(K), &bm, &bn);
    return bm * 1024 + bn;
}

SSG_API int dense_gemm_f16_splitk(const void *A, const void *Wt, void *C, int64_t M, int64_t N, int64_t K,
                                  int32_t splits, void *ws, int64_t ws_bytes, void *stream) {
    return split_run("dense_gemm_f16_splitk", 0, A, Wt, nullptr, nullptr, nullptr, C, 0, M, N, K, splits, ws,
                     ws_bytes, stream);
}

SSG_API int w24_gemm_f16_splitk(const void *A, const void *vals, const uint32_t *meta, void *C, int64_t M, int64_t N,
                                int64_t K, int32_t splits, void *ws, int64_t ws_bytes, void *stream) {
    return split_run("w24_gemm_f16_splitk", 1, A, vals, meta, nullptr, nullptr, C, 0, M, N, K, splits, ws, ws_bytes,
                     stream);
}

SSG_API int dense_gemm_i8_splitk(const int8_t *A, const int8_t *Wt, const float *scale, const float *bias, void *C,
                                 int32_t out_type, int64_t M, int64_t N, int64_t K, int32_t splits, void *ws,
                                 int64_t ws_bytes, void *stream) {
    return split_run("dense_gemm_i8_splitk", 2, A, Wt, nullptr, scale, bias, C, out_type, M, N, K, splits, ws,
                     ws_bytes, stream);
}

SSG_API int w24_gemm_i8_splitk(const int8_t *A, const int8_t *vals, const uint32_t *meta, const float *scale,
                               const float *bias, void *C, int32_t out_type, int64_t M, int64_t N, int64_t K,
                               int32_t splits, void *ws, int64_t ws_bytes, void *stream) {
    return split_run("w24_gemm_i8_splitk", 3, A, vals, meta, scale, bias, C, out_type, M, N, K, splits, ws, ws_bytes,
                     stream);
}

// ---- allocation-free split K.  The partial accumulators live in a
// file-scope device array (one copy per GPU, allocated with the code object
// when the library's kernels are first loaded on that GPU and held until the
// process ends).  In host code `scratch` names a host-side stand-in, so its
// device address is looked up once per device with hipGetSymbolAddress and
// only that address is passed to kernels.
static __device__ __align__(256) uint8_t scratch[SSG_STATIC_SCRATCH_BYTES];

namespace {

std::mutex g_scratch_mu;
void *g_scratch_dev[kMaxDevices] = {nullptr};

// The current device's address of `scratch` (looked up on the first call on
// that device, with the device current).
int scratch_address(void **out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return ssg::fail(SSG_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
    if (dev < 0 || dev >= kMaxDevices) return ssg::fail(SSG_ENODEV, "device id %d out of range", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p)
            return ssg::fail(SSG_EHIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return SSG_OK;
}

}  // namespace

SSG_API int w24_gemm_f16_splitk_static(const void *A, const void *vals, const uint32_t *meta, void *C, int64_t M,
                                       int64_t N, int64_t K, int32_t splits, void *stream) {
    const char *fn = "w24_gemm_f16_splitk_static";
    // shapes first (so the byte count below cannot overflow), then the scratch limit
    int rc = check_gemm(fn, A, vals, C, M, N, K, 64, 64);
    if (rc) return rc;
    const int stages = ssg::gemm_k_stages(1, int(K));
    if (splits < 1 || splits > 64 || stages % splits)
        return ssg::fail(SSG_EINVAL, "%s: splits=%d must be in 1..64 and divide the %d K stages", fn, int(splits),
                         stages);
    if (splits > 1 && M > 0) {
        const int64_t per_split = M * N * 4;  // M, N < 2^31 and M * N / 4096 < 2^31
        if (per_split > int64_t(SSG_STATIC_SCRATCH_BYTES) / splits)
            return ssg::fail(SSG_EINVAL, "%s: splits * M * N * 4 = %d * %lld bytes exceeds the %d-byte static "
                             "scratch (use w24_gemm_f16_splitk with a workspace)", fn, int(splits),
                             (long long)per_split, int(SSG_STATIC_SCRATCH_BYTES));
    }
    void *ws = nullptr;
    if (splits > 1 && M > 0) {
        if ((rc = check_device())) return rc;
        if ((rc = scratch_address(&ws))) return rc;
    }
    return split_run(fn, 1, A, vals, meta, nullptr, nullptr, C, 0, M, N, K, splits, ws,
                     int64_t(SSG_STATIC_SCRATCH_BYTES), stream);
}

namespace {

int tw_run(const char *fn, const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
           const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr, const int32_t *tile_order, int32_t T,
           int32_t G, int32_t t_first, int32_t t_count, int32_t flags, void *C, int64_t M, int64_t N, int64_t K,
           void *stream) {
    if (M < 0 || N <= 0 || K <= 0 || !fits_int(M) || !fits_int(N) || !fits_int(K))
        return ssg::fail(SSG_EINVAL, "%s: bad shape M=%lld N=%lld K=%lld", fn, (long long)M, (long long)N,
                         (long long)K);
    if (G <= 0 || G % 16 || G > 256)
        return ssg::fail(SSG_EINVAL, "%s: G=%d must be a positive multiple of 16, at most 256", fn, G);
    if (N % G) return ssg::fail(SSG_EINVAL, "%s: N=%lld must be a multiple of G=%d", fn, (long long)N, G);
    if (T != N / G) return ssg::fail(SSG_EINVAL, "%s: T=%d must equal N/G=%lld", fn, T, (long long)(N / G));
    if (t_first < 0 || t_count < 1 || int64_t(t_first) + t_count > T)
        return ssg::fail(SSG_EINVAL, "%s: tile range [%d, %d + %d) outside [0, %d)", fn, t_first, t_first, t_count, T);
    if (flags & ~(SSG_TW_OUT_T | SSG_TW_A_ROWMAJOR | SSG_TW_NARROW))
        return ssg::fail(SSG_EINVAL, "%s: unknown flags 0x%x", fn, flags);
    if (!fits_int((M + 127) / 128 * int64_t(t_count))) return ssg::fail(SSG_EINVAL, "%s: too many work items", fn);
    if (M == 0) {
        ssg::clear_error();
        return SSG_OK;
    }
    if (!At || !C || !v_ptr || !k_ptr || !n_ptr || !tile_order || !offset_k || !offset_n || !vals)
        return ssg::fail(SSG_EINVAL, "%s: null pointer", fn);
    if (!ssg::aligned16(At) || !ssg::aligned16(C) || !ssg::aligned16(vals))
        return ssg::fail(SSG_EINVAL, "%s: At, vals and C must be 16-byte aligned", fn);
    int rc = check_device();
    if (rc) return rc;
    return launched(ssg::launch_tw_f16(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, t_first,
                                       t_count, G, (flags & SSG_TW_OUT_T) != 0, (flags & SSG_TW_A_ROWMAJOR) != 0,
                                       (flags & SSG_TW_NARROW) != 0, C, int(M), int(N), int(K), hipStream_t(stream)),
                    fn);
}

}  // namespace

SSG_API int tw_gemm_f16(const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
                        const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr, const int32_t *tile_order,
                        int32_t T, int32_t G, void *C, int64_t M, int64_t N, int64_t K, void *stream) {
    return tw_run("tw_gemm_f16", At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G, 0, T, 0, C, M,
                  N, K, stream);
}

SSG_API int tw_gemm_f16_ex(const void *At, const void *vals, const int32_t *offset_k, const int32_t *offset_n,
                           const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr,
                           const int32_t *tile_order, int32_t T, int32_t G, int32_t t_first, int32_t t_count,
                           int32_t flags, void *C, int64_t M, int64_t N, int64_t K, void *stream) {
    return tw_run("tw_gemm_f16_ex", At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G, t_first,
                  t_count, flags, C, M, N, K, stream);
}

SSG_API int tw_gemm_i8(const int8_t *At, const int8_t *vals, const int32_t *offset_k, const int32_t *offset_n,
                       const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr, const int32_t *tile_order,
                       int32_t T, int32_t G, const float *scale, const float *bias, void *C, int32_t out_type,
                       int64_t M, int64_t N, int64_t K, void *stream) {
    const char *fn = "tw_gemm_i8";
    if (M < 0 || N <= 0 || K <= 0 || !fits_int(M) || !fits_int(N) || !fits_int(K))
        return ssg::fail(SSG_EINVAL, "%s: bad shape M=%lld N=%lld K=%lld", fn, (long long)M, (long long)N,
                         (long long)K);
    if (G <= 0 || G % 16 || G > 256)
        return ssg::fail(SSG_EINVAL, "%s: G=%d must be a positive multiple of 16, at most 256", fn, G);
    if (N % G) return ssg::fail(SSG_EINVAL, "%s: N=%lld must be a multiple of G=%d", fn, (long long)N, G);
    if (T != N / G) return ssg::fail(SSG_EINVAL, "%s: T=%d must equal N/G=%lld", fn, T, (long long)(N / G));
    if (!fits_int((M + 127) / 128 * int64_t(T))) return ssg::fail(SSG_EINVAL, "%s: too many work items", fn);
    int rc = check_i8_epilogue(fn, scale, bias, out_type);
    if (rc) return rc;
    if (M == 0) {
        ssg::clear_error();
        return SSG_OK;
    }
    if (!At || !C || !v_ptr || !k_ptr || !n_ptr || !tile_order || !offset_k || !offset_n || !vals)
        return ssg::fail(SSG_EINVAL, "%s: null pointer", fn);
    if (!ssg::aligned16(At) || !ssg::aligned16(C) || !ssg::aligned16(vals))
        return ssg::fail(SSG_EINVAL, "%s: At, vals and C must be 16-byte aligned", fn);
    if ((rc = check_device())) return rc;
    return launched(ssg::launch_tw_i8(At, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order, T, G, scale,
                                      bias, C, out_type, int(M), int(N), hipStream_t(stream)),
                    fn);
}

SSG_API int ssg_transpose_f16(const void *A, void *At, int64_t M, int64_t K, void *stream) {
    const char *fn = "ssg_transpose_f16";
    if (M < 0 || K <= 0 || !fits_int(M) || !fits_int(K) || M % 8 || K % 8)
        return ssg::fail(SSG_EINVAL, "%s: M=%lld K=%lld must be multiples of 8 (K > 0)", fn, (long long)M,
                         (long long)K);
    if (M == 0) {
        ssg::clear_error();
        return SSG_OK;
    }
    if (!A || !At || !ssg::aligned16(A) || !ssg::aligned16(At))
        return ssg::fail(SSG_EINVAL, "%s: pointers must be non-null and 16-byte aligned", fn);
    int rc = check_device();
    if (rc) return rc;
    return launched(ssg::launch_transpose_f16(A, At, int(M), int(K), hipStream_t(stream)), fn);
}
