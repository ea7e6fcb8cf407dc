// ssm_step.hip -- one decode step for every (batch, head).
//
// Generation runs the model one token at a time on a fixed-size state (page
// "State Space Model", section "Un sistema che riassume il passato", end of
// the water-tank passage; page tech.tersel.eu, section "Porownanie zlozonosci
// obliczeniowej i zachowania pamieci": constant memory per generated token):
//     a = exp(dt A_h);  state[p][n] = a state[p][n] + w x[p] B[n];
//     y[p] = sum_n C[n] state[p][n] + D_h x[p]
// with input weight w = dt, or the exact zero-order hold expm1(dt A_h) / A_h
// (ssm_step_zoh; page "State Space Models (SSM)", section "Come funzionano
// gli SSM").
//
// The state ([batch][H][P][N] fp32) is read and written once; everything else
// is tiny, so the kernel is an HBM stream (non-temporal state accesses: the
// state of a large batch does not stay in cache from one step to the next).  One workgroup per (batch, head):
// NV = N/4 lanes cover one row p with float4 accesses (so a wave reads whole
// 512-byte rows for N = 128), 256/NV rows are in flight per pass, and each
// thread issues the loads of all its rows before using any of them.  The
// read-out sum over n is a butterfly over the NV lanes of a row.
#include "device_common.h"
#include "launchers.h"

namespace ssd {

template <typename T, int NV, int RPT>
__global__ __launch_bounds__(256) void ssm_step_vec_kernel(float* __restrict__ state,
                                                           const T* __restrict__ x,
                                                           const float* __restrict__ dt,
                                                           const float* __restrict__ A,
                                                           const T* __restrict__ Bm,
                                                           const T* __restrict__ Cm,
                                                           const float* __restrict__ D,
                                                           T* __restrict__ y, int H, int P, int N,
                                                           int hpg, int G, int zoh) {
    constexpr int RPP = 256 / NV;  // rows per pass
    const int bh = blockIdx.x;
    const int b = bh / H, h = bh - b * H, g = h / hpg;
    const int n4 = threadIdx.x % NV;
    const int r0 = threadIdx.x / NV;
    const float d = dt[bh];
    const float a = expf(d * A[h]);
    const float w = zoh ? zoh_weight(d, A[h]) : d;   // input weight
    const float Dh = D ? D[h] : 0.0f;

    const int64_t bc = ((int64_t)b * G + g) * N + 4 * n4;
    float bv[4], cv[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        bv[e] = Elem<T>::load(Bm, bc + e);
        cv[e] = Elem<T>::load(Cm, bc + e);
    }
    float* st = state + (int64_t)bh * P * N + 4 * n4;
    const T* xr = x + (int64_t)bh * P;
    T* yr = y + (int64_t)bh * P;

    for (int p0 = r0; p0 < P; p0 += RPP * RPT) {
        // Loads are unconditional (rows past P re-read row P - 1 and are
        // never stored): a load under a branch makes the compiler wait for it
        // at the join, which would issue the rows one at a time.
        float4 s[RPT];
        float xv[RPT];
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int pl = min(p0 + k * RPP, P - 1);
            const f32x4 t = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(st + (int64_t)pl * N));
            s[k] = make_float4(t[0], t[1], t[2], t[3]);
            xv[k] = Elem<T>::load(xr, pl);
        }
#pragma unroll
        for (int k = 0; k < RPT; ++k) {
            const int p = p0 + k * RPP;
            const float u = w * xv[k];
            float4 v = s[k];
            v.x = a * v.x + u * bv[0];
            v.y = a * v.y + u * bv[1];
            v.z = a * v.z + u * bv[2];
            v.w = a * v.w + u * bv[3];
            float part = cv[0] * v.x + cv[1] * v.y + cv[2] * v.z + cv[3] * v.w;
#pragma unroll
            for (int off = NV / 2; off >= 1; off >>= 1) part += __shfl_xor(part, off, 64);
            if (p < P) {
                const f32x4 tv = {v.x, v.y, v.z, v.w};
                __builtin_nontemporal_store(tv, reinterpret_cast<f32x4*>(st + (int64_t)p * N));
                if (n4 == 0) Elem<T>::store(yr, p, part + Dh * xv[k]);
            }
        }
    }
}

// Any P, N: one thread per (batch, head, p), serial over n.  Used only for
// shapes the vector kernel does not cover.
template <typename T>
__global__ __launch_bounds__(256) void ssm_step_generic_kernel(
    float* __restrict__ state, const T* __restrict__ x, const float* __restrict__ dt,
    const float* __restrict__ A, const T* __restrict__ Bm, const T* __restrict__ Cm,
    const float* __restrict__ D, T* __restrict__ y, int64_t rows, int H, int P, int N, int hpg,
    int G, int zoh) {
    const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (r >= rows) return;
    const int64_t bh = r / P;
    const int b = (int)(bh / H), h = (int)(bh % H), g = h / hpg;
    const float d = dt[bh];
    const float a = expf(d * A[h]);
    const float xp = Elem<T>::load(x, r);
    const float u = (zoh ? zoh_weight(d, A[h]) : d) * xp;
    const int64_t bc = ((int64_t)b * G + g) * N;
    float* st = state + r * N;
    float acc = 0.0f;
    for (int n = 0; n < N; ++n) {
        const float v = a * st[n] + u * Elem<T>::load(Bm, bc + n);
        st[n] = v;
        acc += Elem<T>::load(Cm, bc + n) * v;
    }
    Elem<T>::store(y, r, acc + (D ? D[h] : 0.0f) * xp);
}

bool ssm_step_supported(int64_t P, int64_t N) { return P >= 1 && P <= 1024 && N >= 1 && N <= 1024; }

template <typename T, int NV>
static void launch_vec(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G, float* state,
                       const void* x, const float* dt, const float* A, const void* B,
                       const void* C, const float* D, void* y, hipStream_t stream, int zoh) {
    ssm_step_vec_kernel<T, NV, 8><<<(unsigned)(batch * H), 256, 0, stream>>>(
        state, static_cast<const T*>(x), dt, A, static_cast<const T*>(B),
        static_cast<const T*>(C), D, static_cast<T*>(y), (int)H, (int)P, (int)N, (int)(H / G),
        (int)G, zoh);
}

template <typename T>
static void launch_typed(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G,
                         float* state, const void* x, const float* dt, const float* A,
                         const void* B, const void* C, const float* D, void* y,
                         hipStream_t stream, int zoh) {
    switch (N) {
        case 4: launch_vec<T, 1>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh); return;
        case 8: launch_vec<T, 2>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh); return;
        case 16: launch_vec<T, 4>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh); return;
        case 32: launch_vec<T, 8>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh); return;
        case 64: launch_vec<T, 16>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh); return;
        case 128: launch_vec<T, 32>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh); return;
        case 256: launch_vec<T, 64>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh); return;
        default: break;
    }
    const int64_t rows = batch * H * P;
    ssm_step_generic_kernel<T><<<(unsigned)((rows + 255) / 256), 256, 0, stream>>>(
        state, static_cast<const T*>(x), dt, A, static_cast<const T*>(B),
        static_cast<const T*>(C), D, static_cast<T*>(y), rows, (int)H, (int)P, (int)N,
        (int)(H / G), (int)G, zoh);
}

hipError_t launch_ssm_step(int64_t batch, int64_t H, int64_t P, int64_t N, int64_t G,
                           int32_t dtype, float* state, const void* x, const float* dt,
                           const float* A, const void* B, const void* C, const float* D,
                           void* y, hipStream_t stream, bool zoh) {
    if (dtype == 1)
        launch_typed<bf16_t>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh ? 1 : 0);
    else
        launch_typed<float>(batch, H, P, N, G, state, x, dt, A, B, C, D, y, stream, zoh ? 1 : 0);
    return hipGetLastError();
}

}  // namespace ssd
