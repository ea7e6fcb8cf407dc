// layer.hip -- the steps a Mamba block puts around the selective scan.
//
// Each block wraps the selective SSM with a short convolution and a SiLU gate,
// and Delta, B, C are functions of the current token (page "State Space Models
// (SSM)", ultralytics.com glossary, section "Da S4 a Mamba").  Read plainly:
//
//   layer_in:  u[t, c] = silu(bias[c] + sum_k w[c, k] xbc[t - (K - 1) + k, c])
//              (depthwise causal K-tap convolution, zeros before the first
//              token), split by channel into x [.., H, P], B [.., G, N] and
//              C [.., G, N]; dt = softplus(dt_raw + dt_bias[h]).
//   layer_out: out = y * silu(z).
//
// Both are pure streams (every input read once, every output written once).
// The vector convolution kernel gives each thread 8 consecutive channels and a
// run of kLayerRun tokens: the K - 1 previous inputs stay in registers as the
// thread walks its tokens, and each run re-reads only its K - 1 halo tokens
// (about 5% more reads at K = 4).  The step sizes ride in the same launch, one
// extra block per run.
#include <cmath>

#include "device_common.h"
#include "launchers.h"

namespace ssd {

namespace {

// silu_f (device_common.h): e^-v overflows to +inf for v < -88, and
// rcp(inf) = 0 gives -0.
// log(1 + e^v) without overflow: max(v, 0) + log1p(e^-|v|)
__device__ __forceinline__ float softplus_f(float v) { return fmaxf(v, 0.0f) + log1pf(expf(-fabsf(v))); }

typedef uint32_t u32x4e __attribute__((ext_vector_type(4)));

// 8 elements of T: raw 16- or 32-byte loads (optionally non-temporal, for
// data read once), unpacking to fp32, and stores from fp32.
template <typename T>
struct Vec8;
template <>
struct Vec8<bf16_t> {
    struct Raw { uint4 u; };
    __device__ __forceinline__ static Raw load_raw(const bf16_t* p) {
        return Raw{*reinterpret_cast<const uint4*>(p)};
    }
    __device__ __forceinline__ static Raw load_raw_nt(const bf16_t* p) {
        const u32x4e v = __builtin_nontemporal_load(reinterpret_cast<const u32x4e*>(p));
        return Raw{make_uint4(v.x, v.y, v.z, v.w)};
    }
    __device__ __forceinline__ static void store_nt(bf16_t* p, const float (&v)[8]) {
        const u32x4e u = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]), pack_bf16x2(v[4], v[5]),
                          pack_bf16x2(v[6], v[7])};
        __builtin_nontemporal_store(u, reinterpret_cast<u32x4e*>(p));
    }
    __device__ __forceinline__ static void unpack(const Raw& r, float (&v)[8]) {
        const uint32_t w[4] = {r.u.x, r.u.y, r.u.z, r.u.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
            v[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
        }
    }
    __device__ __forceinline__ static void load(const bf16_t* p, float (&v)[8]) {
        unpack(load_raw(p), v);
    }
    __device__ __forceinline__ static void store(bf16_t* p, const float (&v)[8]) {
        uint4 u;
        u.x = pack_bf16x2(v[0], v[1]);
        u.y = pack_bf16x2(v[2], v[3]);
        u.z = pack_bf16x2(v[4], v[5]);
        u.w = pack_bf16x2(v[6], v[7]);
        *reinterpret_cast<uint4*>(p) = u;
    }
};
template <>
struct Vec8<float> {
    struct Raw { float4 a, b; };
    __device__ __forceinline__ static Raw load_raw(const float* p) {
        return Raw{*reinterpret_cast<const float4*>(p), *reinterpret_cast<const float4*>(p + 4)};
    }
    __device__ __forceinline__ static Raw load_raw_nt(const float* p) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + 4));
        return Raw{make_float4(a[0], a[1], a[2], a[3]), make_float4(b[0], b[1], b[2], b[3])};
    }
    __device__ __forceinline__ static void store_nt(float* p, const float (&v)[8]) {
        const f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        __builtin_nontemporal_store(a, reinterpret_cast<f32x4*>(p));
        __builtin_nontemporal_store(b, reinterpret_cast<f32x4*>(p + 4));
    }
    __device__ __forceinline__ static void unpack(const Raw& r, float (&v)[8]) {
        v[0] = r.a.x; v[1] = r.a.y; v[2] = r.a.z; v[3] = r.a.w;
        v[4] = r.b.x; v[5] = r.b.y; v[6] = r.b.z; v[7] = r.b.w;
    }
    __device__ __forceinline__ static void load(const float* p, float (&v)[8]) {
        unpack(load_raw(p), v);
    }
    __device__ __forceinline__ static void store(float* p, const float (&v)[8]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
};

constexpr int kLayerRun = 64;      // tokens per thread in the vector convolution
constexpr int kLayerThreads = 256; // threads (8-channel groups) per convolution block

}  // namespace

// 8 channels per thread; channel groups never straddle x / B / C (H P and
// G N are multiples of 8).  grid: (runs, channel groups / kLayerThreads + 1,
// batch); the last y-block of each run computes the run's step sizes instead.
template <typename T, int K>
__global__ __launch_bounds__(256) void layer_in_vec_kernel(const T* __restrict__ xbc,
                                                           const float* __restrict__ w,
                                                           const float* __restrict__ bias,
                                                           T* __restrict__ x, T* __restrict__ Bm,
                                                           T* __restrict__ Cm,
                                                           const float* __restrict__ dt_raw,
                                                           const float* __restrict__ dt_bias,
                                                           float* __restrict__ dt, int L, int Cd,
                                                           int HP, int GN, int H) {
    if (blockIdx.y == gridDim.y - 1) {   // the run's step sizes: dt = softplus(dt_raw + dt_bias)
        const int t0 = blockIdx.x * kLayerRun, t1 = min(t0 + kLayerRun, L);
        const int64_t base = ((int64_t)blockIdx.z * L + t0) * H;
        const int n = (t1 - t0) * H;
        for (int i = threadIdx.x; i < n; i += kLayerThreads)
            dt[base + i] = softplus_f(dt_raw[base + i] + (dt_bias ? dt_bias[i % H] : 0.0f));
        return;
    }
    const int cg = blockIdx.y * kLayerThreads + threadIdx.x;
    const int c0 = 8 * cg;
    if (c0 >= Cd) return;
    const int b = blockIdx.z;
    const int t0 = blockIdx.x * kLayerRun, t1 = min(t0 + kLayerRun, L);

    float wr[8][K], br[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
#pragma unroll
        for (int k = 0; k < K; ++k) wr[i][k] = w[(int64_t)(c0 + i) * K + k];
        br[i] = bias ? bias[c0 + i] : 0.0f;
    }
    T* dst;
    int dc, ds;
    if (c0 < HP) { dst = x; dc = c0; ds = HP; }
    else if (c0 < HP + GN) { dst = Bm; dc = c0 - HP; ds = GN; }
    else { dst = Cm; dc = c0 - HP - GN; ds = GN; }
    const T* src = xbc + (int64_t)b * L * Cd + c0;
    dst += (int64_t)b * L * ds + dc;

    // the K - 1 inputs before the run (zeros before the first token)
    float win[K > 1 ? K - 1 : 1][8];
#pragma unroll
    for (int k = 0; k < K - 1; ++k) {
        const int t = t0 - (K - 1) + k;
        if (t >= 0) Vec8<T>::load(src + (int64_t)t * Cd, win[k]);
        else {
#pragma unroll
            for (int i = 0; i < 8; ++i) win[k][i] = 0.0f;
        }
    }
    // one output token from its input v and the window; then slide the window
    auto emit = [&](const float (&v)[8], int t) {
        float o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            float a = br[i];
#pragma unroll
            for (int k = 0; k < K - 1; ++k) a += wr[i][k] * win[k][i];
            a += wr[i][K - 1] * v[i];
            o[i] = silu_f(a);
        }
        if (t < t1) Vec8<T>::store(dst + (int64_t)t * ds, o);
#pragma unroll
        for (int k = 0; k + 1 < K - 1; ++k)
#pragma unroll
            for (int i = 0; i < 8; ++i) win[k][i] = win[k + 1][i];
        if (K > 1) {
#pragma unroll
            for (int i = 0; i < 8; ++i) win[K > 1 ? K - 2 : 0][i] = v[i];
        }
    };
    // The run goes in NG groups of U tokens, double-buffered: the U loads of
    // group g + 1 are issued (in token order, pinned there by the scheduling
    // barriers) before group g is computed, so a wave always has a group in
    // flight.  Loads past the end of a ragged last run re-read its last
    // token (always in bounds) and those tokens are not stored; they come
    // after every real token, so the window they disturb is not used again.
    constexpr int U = 16 / sizeof(T);
    constexpr int NG = kLayerRun / U;
    static_assert(kLayerRun % U == 0, "run length");
    typename Vec8<T>::Raw r[2][U];
    auto issue = [&](int g) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = min(t0 + g * U + u, t1 - 1);
            r[g & 1][u] = Vec8<T>::load_raw(src + (int64_t)t * Cd);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    issue(0);
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        if (g + 1 < NG) issue(g + 1);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float v[8];
            Vec8<T>::unpack(r[g & 1][u], v);
            emit(v, t0 + g * U + u);
        }
    }
}

// Any channel count and K <= 8: one thread per (token, channel).
template <typename T>
__global__ __launch_bounds__(256) void layer_in_generic_kernel(const T* __restrict__ xbc,
                                                               const float* __restrict__ w,
                                                               const float* __restrict__ bias,
                                                               T* __restrict__ x, T* __restrict__ Bm,
                                                               T* __restrict__ Cm, int64_t total,
                                                               int L, int Cd, int HP, int GN, int K) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    const int c = (int)(i % Cd);
    const int64_t bt = i / Cd;
    const int t = (int)(bt % L);
    float a = bias ? bias[c] : 0.0f;
    for (int k = 0; k < K; ++k) {
        const int tt = t - (K - 1) + k;
        if (tt >= 0) a += w[(int64_t)c * K + k] * Elem<T>::load(xbc, i - (int64_t)(K - 1 - k) * Cd);
    }
    const float o = silu_f(a);
    if (c < HP) Elem<T>::store(x, bt * HP + c, o);
    else if (c < HP + GN) Elem<T>::store(Bm, bt * GN + (c - HP), o);
    else Elem<T>::store(Cm, bt * GN + (c - HP - GN), o);
}

__global__ __launch_bounds__(256) void layer_dt_kernel(const float* __restrict__ dt_raw,
                                                       const float* __restrict__ dt_bias,
                                                       float* __restrict__ dt, int64_t total, int H) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    dt[i] = softplus_f(dt_raw[i] + (dt_bias ? dt_bias[i % H] : 0.0f));
}

// y and out may be one array (in-place gate), so neither is __restrict__.
// Each thread takes kOutVec 8-element vectors, a block's vectors being
// contiguous and each step of the block coalesced; all loads of a full tile
// are issued before any arithmetic.  Every element is touched once, so full
// tiles use non-temporal loads and stores (172 -> 154 us at the 2.7B shape;
// the same hint on the convolution's input made no difference).
constexpr int kOutVec = 4;
template <typename T>
__global__ __launch_bounds__(256) void layer_out_vec_kernel(const T* y, const T* __restrict__ z,
                                                            T* out, int64_t n8) {
    const int64_t i0 = (int64_t)blockIdx.x * (256 * kOutVec) + threadIdx.x;
    typename Vec8<T>::Raw ry[kOutVec], rz[kOutVec];
    if ((int64_t)(blockIdx.x + 1) * (256 * kOutVec) <= n8) {
#pragma unroll
        for (int v = 0; v < kOutVec; ++v) {
            ry[v] = Vec8<T>::load_raw_nt(y + 8 * (i0 + 256 * v));
            rz[v] = Vec8<T>::load_raw_nt(z + 8 * (i0 + 256 * v));
        }
#pragma unroll
        for (int v = 0; v < kOutVec; ++v) {
            float yv[8], zv[8];
            Vec8<T>::unpack(ry[v], yv);
            Vec8<T>::unpack(rz[v], zv);
#pragma unroll
            for (int k = 0; k < 8; ++k) yv[k] *= silu_f(zv[k]);
            Vec8<T>::store_nt(out + 8 * (i0 + 256 * v), yv);
        }
        return;
    }
    for (int v = 0; v < kOutVec; ++v) {   // the last, partial tile
        const int64_t i = i0 + 256 * v;
        if (i >= n8) return;
        float yv[8], zv[8];
        Vec8<T>::load(y + 8 * i, yv);
        Vec8<T>::load(z + 8 * i, zv);
#pragma unroll
        for (int k = 0; k < 8; ++k) yv[k] *= silu_f(zv[k]);
        Vec8<T>::store(out + 8 * i, yv);
    }
}

template <typename T>
__global__ __launch_bounds__(256) void layer_out_generic_kernel(const T* y, const T* __restrict__ z,
                                                                T* out, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= n) return;
    Elem<T>::store(out, i, Elem<T>::load(y, i) * silu_f(Elem<T>::load(z, i)));
}

// Returns hipSuccess with *dt_done set when the vector kernel also computed dt.
template <typename T>
static hipError_t launch_layer_in_t(int64_t batch, int64_t L, int64_t HP, int64_t GN, int64_t H,
                                    int K, const void* xbc, const float* w, const float* bias,
                                    void* x, void* B, void* C, const float* dt_raw,
                                    const float* dt_bias, float* dt, bool* dt_done,
                                    hipStream_t stream) {
    *dt_done = false;
    const int64_t Cd = HP + 2 * GN;
    const T* s = static_cast<const T*>(xbc);
    T* xo = static_cast<T*>(x);
    T* bo = static_cast<T*>(B);
    T* co = static_cast<T*>(C);
    const bool vec = HP % 8 == 0 && GN % 8 == 0 && ((uintptr_t)xbc | (uintptr_t)x | (uintptr_t)B |
                                                    (uintptr_t)C) % 16 == 0;
    if (vec) {
        dim3 grid((unsigned)((L + kLayerRun - 1) / kLayerRun),
                  (unsigned)((Cd / 8 + kLayerThreads - 1) / kLayerThreads + 1), (unsigned)batch);
        switch (K) {
#define SSD_LAYER_K(k)                                                                    \
    case k:                                                                               \
        layer_in_vec_kernel<T, k><<<grid, kLayerThreads, 0, stream>>>(                    \
            s, w, bias, xo, bo, co, dt_raw, dt_bias, dt, (int)L, (int)Cd, (int)HP, (int)GN, \
            (int)H);                                                                      \
        *dt_done = true;                                                                  \
        return hipGetLastError();
            SSD_LAYER_K(1) SSD_LAYER_K(2) SSD_LAYER_K(3) SSD_LAYER_K(4)
            SSD_LAYER_K(5) SSD_LAYER_K(6) SSD_LAYER_K(7) SSD_LAYER_K(8)
#undef SSD_LAYER_K
            default: break;
        }
    }
    const int64_t total = batch * L * Cd;
    layer_in_generic_kernel<T><<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(
        s, w, bias, xo, bo, co, total, (int)L, (int)Cd, (int)HP, (int)GN, K);
    return hipGetLastError();
}

hipError_t launch_layer_in(int64_t batch, int64_t L, int64_t H, int64_t P, int64_t G, int64_t N,
                           int K, int32_t dtype, const void* xbc, const float* w, const float* bias,
                           const float* dt_raw, const float* dt_bias, void* x, void* B, void* C,
                           float* dt, hipStream_t stream) {
    bool dt_done = false;
    hipError_t e = dtype == 1
        ? launch_layer_in_t<bf16_t>(batch, L, H * P, G * N, H, K, xbc, w, bias, x, B, C, dt_raw,
                                    dt_bias, dt, &dt_done, stream)
        : launch_layer_in_t<float>(batch, L, H * P, G * N, H, K, xbc, w, bias, x, B, C, dt_raw,
                                   dt_bias, dt, &dt_done, stream);
    if (e != hipSuccess || dt_done) return e;
    const int64_t total = batch * L * H;
    layer_dt_kernel<<<(unsigned)((total + 255) / 256), 256, 0, stream>>>(dt_raw, dt_bias, dt, total, (int)H);
    return hipGetLastError();
}

template <typename T>
static void launch_layer_out_t(int64_t n, const void* y, const void* z, void* out, hipStream_t stream) {
    const T* yp = static_cast<const T*>(y);
    const T* zp = static_cast<const T*>(z);
    T* op = static_cast<T*>(out);
    if (n % 8 == 0 && ((uintptr_t)y | (uintptr_t)z | (uintptr_t)out) % 16 == 0) {
        const int64_t n8 = n / 8;
        layer_out_vec_kernel<T><<<(unsigned)((n8 + 256 * kOutVec - 1) / (256 * kOutVec)), 256, 0,
                                  stream>>>(yp, zp, op, n8);
    } else {
        layer_out_generic_kernel<T><<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(yp, zp, op, n);
    }
}

hipError_t launch_layer_out(int64_t n, int32_t dtype, const void* y, const void* z, void* out,
                            hipStream_t stream) {
    if (dtype == 1) launch_layer_out_t<bf16_t>(n, y, z, out, stream);
    else launch_layer_out_t<float>(n, y, z, out, stream);
    return hipGetLastError();
}

}  // namespace ssd
