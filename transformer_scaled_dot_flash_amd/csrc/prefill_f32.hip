// fp32 attention forward (fp32 inputs, fp32 arithmetic), gfx950.
//
// Same method as the bf16 kernels (tiling over keys with the online-softmax
// recurrence and block merge of AIInfraGuide "3.3 Self-Attention机制深入理解",
// sections 7.3 and 12.3), but on fp32 FMA units: bf16 matrix cores cannot
// meet an fp32 accuracy contract.  Used for every fp32 call, prefill and
// decode.
//
// Two kernels, both over the rows (q head within the kv group, query
// position) of one (batch, kv head), so that a decode call (T_q = 1) packs
// the query heads of a kv head into one workgroup and reads that kv head's
// K and V once:
//   * attn_f32_kernel (large problems): 64 rows per workgroup, four threads
//     per row, thread c owning features c, c+4, ... (four different LDS
//     banks); K and V tiles of 32 keys in LDS serve all 64 rows.
//   * attn_f32_row_kernel (small problems, where the time is the length of
//     each thread's dependent chain, not throughput): one wave per row and
//     four rows per workgroup; per 64-key tile each lane scores one key
//     (four partial sums over the features), the tile's maximum and sum are
//     wave reductions, and each lane accumulates the output features lane,
//     lane + 64 from the tile's weights.  Per tile a lane runs about D / 2 +
//     64 dependent steps instead of the 64 rows kernel's 32 (D / 4 + ...)
//     per key.
#include <math.h>

#include "launch.h"

namespace attn {
namespace {

constexpr int kRows = 64;
constexpr int kBNf = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(256) void attn_f32_kernel(const float* __restrict__ Q,
                                                       const float* __restrict__ K,
                                                       const float* __restrict__ V,
                                                       float* __restrict__ O, int H_q, int H_kv,
                                                       int T_q, int T_kv, int n_rt, float scale) {
    constexpr int DQ = D / 4;
    __shared__ __attribute__((aligned(16))) float ks[kBNf * D];
    __shared__ __attribute__((aligned(16))) float vs[kBNf * D];

    const int tid = threadIdx.x;
    const int rl = tid >> 2;
    const int c = tid & 3;
    const int G = H_q / H_kv;
    const int R = G * T_q;
    const int rt = blockIdx.x % n_rt;
    const int unit = blockIdx.x / n_rt;
    const int b = unit / H_kv;
    const int hk = unit - b * H_kv;

    const int r = rt * kRows + rl;
    const bool valid = r < R;
    const int g = valid ? r / T_q : 0;
    const int t = valid ? r - g * T_q : 0;
    const int hq = hk * G + g;
    const int off = T_kv - T_q;

    float q[DQ];
    float o[DQ];
    const float* qp = Q + ((size_t)(b * H_q + hq) * T_q + t) * D + c;
#pragma unroll
    for (int i = 0; i < DQ; ++i) {
        q[i] = valid ? qp[4 * i] : 0.f;
        o[i] = 0.f;
    }

    // Key range of the workgroup: up to the last visible key of its rows.
    const int r_first = rt * kRows;
    const int r_last = min(R, r_first + kRows) - 1;
    const int t_max = (r_first / T_q == r_last / T_q) ? r_last % T_q : T_q - 1;
    const int kv_end = CAUSAL ? min(T_kv, t_max + off + 1) : T_kv;
    const int lim = CAUSAL ? min(T_kv - 1, t + off) : T_kv - 1;

    const float* Kh = K + (size_t)unit * T_kv * D;
    const float* Vh = V + (size_t)unit * T_kv * D;

    float m = -INFINITY;
    float l = 0.f;
    for (int j0 = 0; j0 < kv_end; j0 += kBNf) {
        __syncthreads();
        for (int e = tid; e < kBNf * D / 4; e += 256) {
            const int row = e / (D / 4);
            const int c4 = e - row * (D / 4);
            const int key = j0 + row;
            float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f);
            float4 vv4 = kv4;
            if (key < T_kv) {
                kv4 = *reinterpret_cast<const float4*>(Kh + (size_t)key * D + 4 * c4);
                vv4 = *reinterpret_cast<const float4*>(Vh + (size_t)key * D + 4 * c4);
            }
            *reinterpret_cast<float4*>(ks + row * D + 4 * c4) = kv4;
            *reinterpret_cast<float4*>(vs + row * D + 4 * c4) = vv4;
        }
        __syncthreads();

        float s[kBNf];
        float mt = -INFINITY;
#pragma unroll
        for (int j = 0; j < kBNf; ++j) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < DQ; ++i) part = fmaf(q[i], ks[j * D + 4 * i + c], part);
            part += __shfl_xor(part, 1);
            part += __shfl_xor(part, 2);
            const float x = (j0 + j <= lim) ? part * scale : -INFINITY;
            s[j] = x;
            mt = fmaxf(mt, x);
        }
        const float m_new = fmaxf(m, mt);
        if (m_new == -INFINITY) continue;  // nothing visible yet in this row
        const float alpha = expf(m - m_new);
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < DQ; ++i) o[i] *= alpha;
#pragma unroll
        for (int j = 0; j < kBNf; ++j) {
            const float p = expf(s[j] - m_new);
            psum += p;
#pragma unroll
            for (int i = 0; i < DQ; ++i) o[i] = fmaf(p, vs[j * D + 4 * i + c], o[i]);
        }
        l = l * alpha + psum;
        m = m_new;
    }

    if (valid) {
        const float inv = 1.f / l;
        float* op = O + ((size_t)(b * H_q + hq) * T_q + t) * D + c;
#pragma unroll
        for (int i = 0; i < DQ; ++i) op[4 * i] = o[i] * inv;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_f(const PrefillArgs& a, hipStream_t s) {
    const int G = a.H_q / a.H_kv;
    const long long R = (long long)G * a.T_q;
    const int n_rt = (int)((R + kRows - 1) / kRows);
    const long long grid = (long long)a.B * a.H_kv * n_rt;
    return launch_kernel(attn_f32_kernel<D, CAUSAL>, dim3((unsigned)grid), dim3(256), 0, s,
                         static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                         static_cast<const float*>(a.v), static_cast<float*>(a.o), a.H_q, a.H_kv,
                         a.T_q, a.T_kv, n_rt, a.scale);
}


// Maximum and sum over the 64 lanes of a wave.
__device__ inline float wave_max(float x) {
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) x = fmaxf(x, __shfl_xor(x, sh));
    return x;
}
__device__ inline float wave_sum(float x) {
#pragma unroll
    for (int sh = 32; sh >= 1; sh >>= 1) x += __shfl_xor(x, sh);
    return x;
}

constexpr int kRowsW = 4;   // rows (waves) per workgroup
constexpr int kKT = 64;     // keys per tile: one per lane

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kRowsW) void attn_f32_row_kernel(const float* __restrict__ Q,
                                                                  const float* __restrict__ K,
                                                                  const float* __restrict__ V,
                                                                  float* __restrict__ O, int H_q, int H_kv,
                                                                  int T_q, int T_kv, int n_rt, float scale) {
    constexpr int KP = D + 4;  // padded K row (floats): lane-per-row float4 reads hit distinct banks
    __shared__ __attribute__((aligned(16))) float ks[kKT * KP];
    __shared__ __attribute__((aligned(16))) float vs[kKT * D];
    __shared__ __attribute__((aligned(16))) float qs[kRowsW][D];
    __shared__ __attribute__((aligned(16))) float ps[kRowsW][kKT];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int w = tid >> 6;
    const int G = H_q / H_kv;
    const int R = G * T_q;
    const int rt = blockIdx.x % n_rt;
    const int unit = blockIdx.x / n_rt;
    const int b = unit / H_kv;
    const int hk = unit - b * H_kv;

    const int r = rt * kRowsW + w;
    const bool valid = r < R;
    const int g = valid ? r / T_q : 0;
    const int t = valid ? r - g * T_q : 0;
    const int hq = hk * G + g;
    const int off = T_kv - T_q;

    const float* qp = Q + ((size_t)(b * H_q + hq) * T_q + t) * D;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) qs[w][lane + 64 * i] = valid ? qp[lane + 64 * i] : 0.f;

    // Key range of the workgroup: up to the last visible key of its rows.
    const int r_first = rt * kRowsW;
    const int r_last = min(R, r_first + kRowsW) - 1;
    const int t_max = (r_first / T_q == r_last / T_q) ? r_last % T_q : T_q - 1;
    const int kv_end = CAUSAL ? min(T_kv, t_max + off + 1) : T_kv;
    const int lim = CAUSAL ? min(T_kv - 1, t + off) : T_kv - 1;

    const float* Kh = K + (size_t)unit * T_kv * D;
    const float* Vh = V + (size_t)unit * T_kv * D;

    float o[D / 64];
#pragma unroll
    for (int i = 0; i < D / 64; ++i) o[i] = 0.f;
    float m = -INFINITY;
    float l = 0.f;
    for (int j0 = 0; j0 < kv_end; j0 += kKT) {
        __syncthreads();  // previous tile fully read (and the Q rows written, on the first pass)
        for (int e = tid; e < kKT * D / 4; e += 64 * kRowsW) {
            const int row = e / (D / 4);
            const int c4 = e - row * (D / 4);
            const int key = j0 + row;
            float4 kv4 = make_float4(0.f, 0.f, 0.f, 0.f);
            float4 vv4 = kv4;
            if (key < T_kv) {
                kv4 = *reinterpret_cast<const float4*>(Kh + (size_t)key * D + 4 * c4);
                vv4 = *reinterpret_cast<const float4*>(Vh + (size_t)key * D + 4 * c4);
            }
            *reinterpret_cast<float4*>(ks + row * KP + 4 * c4) = kv4;
            *reinterpret_cast<float4*>(vs + row * D + 4 * c4) = vv4;
        }
        __syncthreads();

        // score of key j0 + lane: four partial sums over the features
        float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
        for (int i = 0; i < D / 4; ++i) {
            const float4 kk = *reinterpret_cast<const float4*>(ks + lane * KP + 4 * i);
            const float4 qq = *reinterpret_cast<const float4*>(&qs[w][4 * i]);
            a0 = fmaf(qq.x, kk.x, a0);
            a1 = fmaf(qq.y, kk.y, a1);
            a2 = fmaf(qq.z, kk.z, a2);
            a3 = fmaf(qq.w, kk.w, a3);
        }
        const float sc = (j0 + lane <= lim) ? ((a0 + a1) + (a2 + a3)) * scale : -INFINITY;
        const float m_new = fmaxf(m, wave_max(sc));
        if (m_new == -INFINITY) continue;  // nothing visible yet in this row (uniform in the wave)
        const float alpha = expf(m - m_new);
        const float p = expf(sc - m_new);
        l = l * alpha + wave_sum(p);
        m = m_new;
        ps[w][lane] = p;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int i = 0; i < D / 64; ++i) o[i] *= alpha;
#pragma unroll 4
        for (int j = 0; j < kKT; j += 4) {
            const float4 pp = *reinterpret_cast<const float4*>(&ps[w][j]);
#pragma unroll
            for (int i = 0; i < D / 64; ++i) {
                const int d = lane + 64 * i;
                o[i] = fmaf(pp.x, vs[(j + 0) * D + d], o[i]);
                o[i] = fmaf(pp.y, vs[(j + 1) * D + d], o[i]);
                o[i] = fmaf(pp.z, vs[(j + 2) * D + d], o[i]);
                o[i] = fmaf(pp.w, vs[(j + 3) * D + d], o[i]);
            }
        }
        __builtin_amdgcn_wave_barrier();  // ps is rewritten by the next tile
    }

    if (valid) {
        const float inv = 1.f / l;
        float* op = O + ((size_t)(b * H_q + hq) * T_q + t) * D;
#pragma unroll
        for (int i = 0; i < D / 64; ++i) op[lane + 64 * i] = o[i] * inv;
    }
}

template <int D, bool CAUSAL>
hipError_t launch_row(const PrefillArgs& a, hipStream_t s) {
    const int G = a.H_q / a.H_kv;
    const long long R = (long long)G * a.T_q;
    const int n_rt = (int)((R + kRowsW - 1) / kRowsW);
    const long long grid = (long long)a.B * a.H_kv * n_rt;
    return launch_kernel(attn_f32_row_kernel<D, CAUSAL>, dim3((unsigned)grid), dim3(64 * kRowsW), 0, s,
                         static_cast<const float*>(a.q), static_cast<const float*>(a.k),
                         static_cast<const float*>(a.v), static_cast<float*>(a.o), a.H_q, a.H_kv,
                         a.T_q, a.T_kv, n_rt, a.scale);
}

}  // namespace

hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s) {
    // Small problems (at most 2^24 (row, key) pairs): one wave per row.
    const long long pairs = (long long)a.B * a.H_q * a.T_q * a.T_kv;
    if (pairs <= (1ll << 24)) {
        if (a.D == 128) return a.causal ? launch_row<128, true>(a, s) : launch_row<128, false>(a, s);
        return a.causal ? launch_row<64, true>(a, s) : launch_row<64, false>(a, s);
    }
    if (a.D == 128) return a.causal ? launch_f<128, true>(a, s) : launch_f<128, false>(a, s);
    return a.causal ? launch_f<64, true>(a, s) : launch_f<64, false>(a, s);
}

}  // namespace attn
