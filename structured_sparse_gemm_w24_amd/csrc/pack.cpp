// Host pack stage: 2:4 compression and tile-wise condensation.
//
// 2:4 -- GPUSQ-ViT ("Boost Vision Transformer with GPU-Friendly Sparsity and
// Quantization", abstract): weights pruned so that each group of four
// consecutive K entries of an output column holds at most two nonzeros.
// The sparse matrix cores consume the two kept values of a group plus their
// 2-bit positions; this file produces exactly that, in the canonical layout
// documented in ssg.h.
//
// Tile-wise -- "Accelerating Sparse DNN Models without Hardware-Support via
// Tile-Wise Sparsity": offline re-organisation of each G-column tile into a
// condensed dense block plus offset_k (kept rows) and offset_n (kept
// columns), read by the run-time GEMM.
#include <algorithm>
#include <cstring>
#include <numeric>
#include <vector>

#include "status.h"

namespace {

// Kept positions of a group given its nonzero mask (bit i = position i).
// Nonzero positions first, topped up with the lowest zero positions, so that
// exactly two distinct positions are kept; returned ascending.
struct Pair {
    uint8_t lo, hi;
};

Pair kept_pair(unsigned mask) {
    uint8_t pos[4];
    int n = 0;
    for (int i = 0; i < 4; ++i)
        if (mask & (1u << i)) pos[n++] = uint8_t(i);
    for (int i = 0; i < 4 && n < 2; ++i)
        if (!(mask & (1u << i))) pos[n++] = uint8_t(i);
    if (pos[0] > pos[1]) std::swap(pos[0], pos[1]);
    return {pos[0], pos[1]};
}

inline bool nonzero(uint16_t h) { return (h & 0x7FFFu) != 0; }  // -0.0 is zero
inline bool nonzero(int8_t v) { return v != 0; }
inline uint16_t canon(uint16_t h) { return nonzero(h) ? h : uint16_t(0); }
inline int8_t canon(int8_t v) { return v; }

template <typename T>
int w24_pack(const T *W, int64_t K, int64_t N, T *vals, uint32_t *meta) {
    if (!W || !vals || !meta) return ssg::fail(SSG_EINVAL, "w24_pack: null pointer");
    if (K <= 0 || N <= 0) return ssg::fail(SSG_EINVAL, "w24_pack: K=%lld N=%lld must be positive",
                                           (long long)K, (long long)N);
    if (K % 4) return ssg::fail(SSG_EINVAL, "w24_pack: K=%lld is not a multiple of 4", (long long)K);
    const int64_t G = K / 4, half = K / 2, words = (K + 31) / 32;
    // Validate first so that nothing is written on failure.
    for (int64_t g = 0; g < G; ++g) {
        const T *r = W + 4 * g * N;
        for (int64_t n = 0; n < N; ++n) {
            int c = nonzero(r[n]) + nonzero(r[N + n]) + nonzero(r[2 * N + n]) + nonzero(r[3 * N + n]);
            if (c > 2)
                return ssg::fail(SSG_ENOT24, "w24_pack: group %lld of column %lld has %d nonzeros",
                                 (long long)g, (long long)n, c);
        }
    }
    Pair table[16];
    for (unsigned m = 0; m < 16; ++m) table[m] = kept_pair(m);
    std::memset(meta, 0, sizeof(uint32_t) * size_t(words) * size_t(N));
    for (int64_t g = 0; g < G; ++g) {
        const T *r = W + 4 * g * N;
        const int64_t j0 = 2 * g;  // first slot of the group
        for (int64_t n = 0; n < N; ++n) {
            const T w[4] = {r[n], r[N + n], r[2 * N + n], r[3 * N + n]};
            unsigned mask = unsigned(nonzero(w[0])) | unsigned(nonzero(w[1])) << 1 |
                            unsigned(nonzero(w[2])) << 2 | unsigned(nonzero(w[3])) << 3;
            const Pair p = table[mask];
            T *v = vals + n * half;
            v[j0] = canon(w[p.lo]);
            v[j0 + 1] = canon(w[p.hi]);
            uint32_t *mw = meta + n * words;
            mw[j0 / 16] |= uint32_t(p.lo) << (2 * (j0 % 16));
            mw[(j0 + 1) / 16] |= uint32_t(p.hi) << (2 * ((j0 + 1) % 16));
        }
    }
    ssg::clear_error();
    return SSG_OK;
}

template <typename T>
int w24_unpack(const T *vals, const uint32_t *meta, int64_t K, int64_t N, T *W) {
    if (!W || !vals || !meta) return ssg::fail(SSG_EINVAL, "w24_unpack: null pointer");
    if (K <= 0 || N <= 0 || K % 4)
        return ssg::fail(SSG_EINVAL, "w24_unpack: bad shape K=%lld N=%lld", (long long)K, (long long)N);
    const int64_t half = K / 2, words = (K + 31) / 32;
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *mw = meta + n * words;
        for (int64_t j = 0; j < half; j += 2) {
            unsigned lo = (mw[j / 16] >> (2 * (j % 16))) & 3u;
            unsigned hi = (mw[(j + 1) / 16] >> (2 * ((j + 1) % 16))) & 3u;
            if (lo >= hi)
                return ssg::fail(SSG_EINVAL, "w24_unpack: column %lld group %lld positions (%u,%u) not ascending",
                                 (long long)n, (long long)(j / 2), lo, hi);
        }
    }
    std::memset(W, 0, sizeof(T) * size_t(K) * size_t(N));
    for (int64_t n = 0; n < N; ++n) {
        const uint32_t *mw = meta + n * words;
        const T *v = vals + n * half;
        for (int64_t j = 0; j < half; ++j) {
            unsigned pos = (mw[j / 16] >> (2 * (j % 16))) & 3u;
            W[(4 * (j / 2) + pos) * N + n] = canon(v[j]);
        }
    }
    ssg::clear_error();
    return SSG_OK;
}

// ---------------------------------------------------------------- tile-wise
struct TileStruct {
    std::vector<std::vector<int32_t>> rows, cols;
};

// Condensed rows are padded to 16 bytes (8 fp16 or 16 int8 elements) so that
// every row of a tile starts 16-byte aligned.
template <typename T>
constexpr int64_t tw_row_align() {
    return 16 / int64_t(sizeof(T));
}
template <typename T>
int64_t tw_ld(int64_t kt) {
    return (kt + tw_row_align<T>() - 1) / tw_row_align<T>() * tw_row_align<T>();
}

template <typename E>
int tw_scan(const E *W, int64_t K, int64_t N, int32_t G, TileStruct &ts, tw_sizes &sz) {
    if (!W) return ssg::fail(SSG_EINVAL, "tw_pack: null W");
    if (K <= 0 || N <= 0 || G <= 0)
        return ssg::fail(SSG_EINVAL, "tw_pack: K=%lld N=%lld G=%d must be positive", (long long)K,
                         (long long)N, G);
    if (K >= (int64_t(1) << 31) || N >= (int64_t(1) << 31))
        return ssg::fail(SSG_EINVAL, "tw_pack: K and N must be < 2^31");
    const int64_t T = (N + G - 1) / G;
    std::vector<uint8_t> rowmark(size_t(T) * size_t(K), 0), colmark(size_t(N), 0);
    for (int64_t k = 0; k < K; ++k) {
        const E *r = W + k * N;
        for (int64_t c = 0; c < N; ++c) {
            if (nonzero(r[c])) {
                colmark[c] = 1;
                rowmark[size_t(c / G) * size_t(K) + size_t(k)] = 1;
            }
        }
    }
    ts.rows.assign(size_t(T), {});
    ts.cols.assign(size_t(T), {});
    int64_t skt = 0, snt = 0, sv = 0;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t k = 0; k < K; ++k)
            if (rowmark[size_t(t) * size_t(K) + size_t(k)]) ts.rows[t].push_back(int32_t(k));
        const int64_t c0 = t * G, c1 = std::min<int64_t>(N, c0 + G);
        for (int64_t c = c0; c < c1; ++c)
            if (colmark[c]) ts.cols[t].push_back(int32_t(c - c0));
        const int64_t kt = int64_t(ts.rows[t].size()), nt = int64_t(ts.cols[t].size());
        skt += kt;
        snt += nt;
        sv += nt * tw_ld<E>(kt);
    }
    if (sv >= (int64_t(1) << 31) || skt >= (int64_t(1) << 31))
        return ssg::fail(SSG_EINVAL, "tw_pack: packed sizes exceed int32 range");
    sz.T = T;
    sz.sum_kt = skt;
    sz.sum_nt = snt;
    sz.vals_elems = sv;
    return SSG_OK;
}


template <typename T>
int tw_pack(const char *fn, const T *W, int64_t K, int64_t N, int32_t G, const tw_sizes *cap, T *vals,
            int32_t *offset_k, int32_t *offset_n, int32_t *v_ptr, int32_t *k_ptr, int32_t *n_ptr,
            int32_t *tile_order) {
    if (!cap || !v_ptr || !k_ptr || !n_ptr || !tile_order) return ssg::fail(SSG_EINVAL, "%s: null pointer", fn);
    TileStruct ts;
    tw_sizes sz{};
    int rc = tw_scan(W, K, N, G, ts, sz);
    if (rc) return rc;
    if (cap->T < sz.T || cap->sum_kt < sz.sum_kt || cap->sum_nt < sz.sum_nt || cap->vals_elems < sz.vals_elems)
        return ssg::fail(SSG_ENOSPC,
                         "%s: capacity (T=%lld kt=%lld nt=%lld vals=%lld) < needed "
                         "(T=%lld kt=%lld nt=%lld vals=%lld)",
                         fn, (long long)cap->T, (long long)cap->sum_kt, (long long)cap->sum_nt,
                         (long long)cap->vals_elems, (long long)sz.T, (long long)sz.sum_kt, (long long)sz.sum_nt,
                         (long long)sz.vals_elems);
    if ((sz.sum_kt && !offset_k) || (sz.sum_nt && !offset_n) || (sz.vals_elems && !vals))
        return ssg::fail(SSG_EINVAL, "%s: null output array", fn);
    const int64_t T_ = sz.T;
    std::vector<int64_t> work(static_cast<size_t>(T_));
    int64_t vp = 0, kp = 0, np = 0;
    v_ptr[0] = k_ptr[0] = n_ptr[0] = 0;
    for (int64_t t = 0; t < T_; ++t) {
        const auto &rows = ts.rows[t];
        const auto &cols = ts.cols[t];
        const int64_t kt = int64_t(rows.size()), nt = int64_t(cols.size());
        const int64_t ld = tw_ld<T>(kt);
        for (int64_t j = 0; j < nt; ++j) {
            T *dst = vals + vp + j * ld;
            const int64_t c = t * int64_t(G) + cols[j];
            for (int64_t kk = 0; kk < kt; ++kk) dst[kk] = canon(W[int64_t(rows[kk]) * N + c]);
            for (int64_t kk = kt; kk < ld; ++kk) dst[kk] = T(0);
        }
        std::copy(rows.begin(), rows.end(), offset_k + kp);
        std::copy(cols.begin(), cols.end(), offset_n + np);
        vp += nt * ld;
        kp += kt;
        np += nt;
        v_ptr[t + 1] = int32_t(vp);
        k_ptr[t + 1] = int32_t(kp);
        n_ptr[t + 1] = int32_t(np);
        work[t] = kt * nt;
    }
    std::vector<int32_t> order(static_cast<size_t>(T_));
    std::iota(order.begin(), order.end(), 0);
    std::stable_sort(order.begin(), order.end(), [&](int32_t a, int32_t b) { return work[a] > work[b]; });
    std::copy(order.begin(), order.end(), tile_order);
    ssg::clear_error();
    return SSG_OK;
}

template <typename T>
int tw_unpack(const char *fn, const T *vals, const int32_t *offset_k, const int32_t *offset_n, const int32_t *v_ptr,
              const int32_t *k_ptr, const int32_t *n_ptr, int64_t K, int64_t N, int32_t G, T *W) {
    if (!W || !v_ptr || !k_ptr || !n_ptr) return ssg::fail(SSG_EINVAL, "%s: null pointer", fn);
    if (K <= 0 || N <= 0 || G <= 0) return ssg::fail(SSG_EINVAL, "%s: bad shape", fn);
    const int64_t T_ = (N + G - 1) / G;
    if (v_ptr[0] != 0 || k_ptr[0] != 0 || n_ptr[0] != 0)
        return ssg::fail(SSG_EINVAL, "%s: prefix sums must start at 0", fn);
    for (int64_t t = 0; t < T_; ++t) {
        const int64_t kt = k_ptr[t + 1] - k_ptr[t], nt = n_ptr[t + 1] - n_ptr[t];
        const int64_t g = std::min<int64_t>(G, N - t * G);
        if (kt < 0 || nt < 0 || v_ptr[t + 1] - v_ptr[t] != nt * tw_ld<T>(kt))
            return ssg::fail(SSG_EINVAL, "%s: inconsistent pointers at tile %lld", fn, (long long)t);
    }
    if ((k_ptr[T_] && !offset_k) || (n_ptr[T_] && !offset_n) || (v_ptr[T_] && !vals))
        return ssg::fail(SSG_EINVAL, "%s: null array with nonzero length", fn);
    for (int64_t t = 0; t < T_; ++t) {
        const int64_t kt = k_ptr[t + 1] - k_ptr[t], nt = n_ptr[t + 1] - n_ptr[t];
        const int64_t g = std::min<int64_t>(G, N - t * G);
        for (int64_t kk = 0; kk < kt; ++kk)
            if (offset_k[k_ptr[t] + kk] < 0 || offset_k[k_ptr[t] + kk] >= K)
                return ssg::fail(SSG_EINVAL, "%s: offset_k out of range in tile %lld", fn, (long long)t);
        for (int64_t j = 0; j < nt; ++j)
            if (offset_n[n_ptr[t] + j] < 0 || offset_n[n_ptr[t] + j] >= g)
                return ssg::fail(SSG_EINVAL, "%s: offset_n out of range in tile %lld", fn, (long long)t);
    }
    std::memset(W, 0, sizeof(T) * size_t(K) * size_t(N));
    for (int64_t t = 0; t < T_; ++t) {
        const int64_t kt = k_ptr[t + 1] - k_ptr[t], nt = n_ptr[t + 1] - n_ptr[t];
        const int64_t ld = tw_ld<T>(kt);
        for (int64_t j = 0; j < nt; ++j) {
            const int64_t c = t * int64_t(G) + offset_n[n_ptr[t] + j];
            const T *src = vals + v_ptr[t] + j * ld;
            for (int64_t kk = 0; kk < kt; ++kk) W[int64_t(offset_k[k_ptr[t] + kk]) * N + c] = canon(src[kk]);
        }
    }
    ssg::clear_error();
    return SSG_OK;
}

template <typename T>
int tw_query(const T *W, int64_t K, int64_t N, int32_t G, tw_sizes *out) {
    if (!out) return ssg::fail(SSG_EINVAL, "tw_pack_query: null out");
    TileStruct ts;
    tw_sizes sz{};
    int rc = tw_scan(W, K, N, G, ts, sz);
    if (rc) return rc;
    *out = sz;
    ssg::clear_error();
    return SSG_OK;
}

}  // namespace

SSG_API int w24_pack_f16(const uint16_t *W, int64_t K, int64_t N, uint16_t *vals, uint32_t *meta) {
    return w24_pack<uint16_t>(W, K, N, vals, meta);
}

SSG_API int w24_pack_i8(const int8_t *W, int64_t K, int64_t N, int8_t *vals, uint32_t *meta) {
    return w24_pack<int8_t>(W, K, N, vals, meta);
}

SSG_API int w24_unpack_f16(const uint16_t *vals, const uint32_t *meta, int64_t K, int64_t N, uint16_t *W) {
    return w24_unpack<uint16_t>(vals, meta, K, N, W);
}

SSG_API int w24_unpack_i8(const int8_t *vals, const uint32_t *meta, int64_t K, int64_t N, int8_t *W) {
    return w24_unpack<int8_t>(vals, meta, K, N, W);
}

SSG_API int tw_pack_query(const uint16_t *W, int64_t K, int64_t N, int32_t G, tw_sizes *out) {
    return tw_query(W, K, N, G, out);
}

SSG_API int tw_pack_query_i8(const int8_t *W, int64_t K, int64_t N, int32_t G, tw_sizes *out) {
    return tw_query(W, K, N, G, out);
}

SSG_API int tw_pack_f16(const uint16_t *W, int64_t K, int64_t N, int32_t G, const tw_sizes *cap,
                        uint16_t *vals, int32_t *offset_k, int32_t *offset_n, int32_t *v_ptr,
                        int32_t *k_ptr, int32_t *n_ptr, int32_t *tile_order) {
    return tw_pack("tw_pack_f16", W, K, N, G, cap, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order);
}

SSG_API int tw_pack_i8(const int8_t *W, int64_t K, int64_t N, int32_t G, const tw_sizes *cap, int8_t *vals,
                       int32_t *offset_k, int32_t *offset_n, int32_t *v_ptr, int32_t *k_ptr, int32_t *n_ptr,
                       int32_t *tile_order) {
    return tw_pack("tw_pack_i8", W, K, N, G, cap, vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, tile_order);
}

SSG_API int tw_unpack_f16(const uint16_t *vals, const int32_t *offset_k, const int32_t *offset_n,
                          const int32_t *v_ptr, const int32_t *k_ptr, const int32_t *n_ptr,
                          int64_t K, int64_t N, int32_t G, uint16_t *W) {
    return tw_unpack("tw_unpack_f16", vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, K, N, G, W);
}

SSG_API int tw_unpack_i8(const int8_t *vals, const int32_t *offset_k, const int32_t *offset_n, const int32_t *v_ptr,
                         const int32_t *k_ptr, const int32_t *n_ptr, int64_t K, int64_t N, int32_t G, int8_t *W) {
    return tw_unpack("tw_unpack_i8", vals, offset_k, offset_n, v_ptr, k_ptr, n_ptr, K, N, G, W);
}
