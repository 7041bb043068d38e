// Host-side launch arguments of the kernels and the launch helper, shared by
// the kernel sources' launchers and the C ABI layer (attn_api.hip).
#pragma once

#include "kernel_common.h"

namespace attn {

struct PrefillArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int B, H_q, H_kv, T_q, T_kv, D;
    int causal;
    float scale;       // multiplier of the raw dot product
    float scale_log2;  // scale * log2(e), rounded to float
    float c_log2;      // |scale| * log2(e), >= FLT_MIN (0 becomes FLT_MIN: same weights)
    int neg_q;         // 1 when scale < 0: the kernels flip Q's sign instead
    int window;        // causal sliding window in keys (0: none)
    const int* cu_q;   // packed batch: [B + 1] row offsets of each sequence's
    const int* cu_k;   //   queries / keys (nullptr: contiguous [B][H][T][D])
    int total_q;       // packed batch: rows of q (picks the launch shape)
};

struct DecodeArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    int B, H_q, H_kv, T_kv, D;
    float c_log2;  // |scale| * log2(e), >= FLT_MIN
    int neg_q;     // 1 when scale < 0 (Q's sign is flipped instead)
    int n_splits;        // effective split count (no split is empty)
    int keys_per_split;  // multiple of 32
    float* ws_o;         // [B][H_q][n_splits][D]  unnormalised partial outputs
    float* ws_ml;        // [B][H_q][n_splits][2]  (running max in log2 units, sum)
    PagedKV paged;       // paged cache (T_kv = max_pages * page_size), or all zero
};

struct QkvArgs {
    const void* x;   // [M][d_model]
    const void* w;   // [N][d_model], N = (H_q + 2 H_kv) D
    void* q;         // [B][H_q][T][D]
    void* k;         // [B][H_kv][T][D]
    void* v;         // [B][H_kv][T][D]
    int M, N, d_model, T, H_q, H_kv, D;
};

// Launchers return the HIP status of the launch call itself.
hipError_t launch_prefill_bf16(const PrefillArgs& a, hipStream_t s);
hipError_t launch_prefill_f32(const PrefillArgs& a, hipStream_t s);
hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t s);
hipError_t launch_qkv_bf16(const QkvArgs& a, hipStream_t s);

template <typename Tup, size_t... I>
inline void fill_ptrs(Tup& t, void** p, std::index_sequence<I...>) {
    ((p[I] = static_cast<void*>(&std::get<I>(t))), ...);
}

// Launch a kernel and return the launch's own error code (no reliance on the
// thread's sticky last-error state).
template <typename... KArgs, typename... Args>
inline hipError_t launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t shmem,
                                hipStream_t s, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count mismatch");
    auto tup = std::make_tuple(static_cast<KArgs>(args)...);
    void* ptrs[sizeof...(KArgs) > 0 ? sizeof...(KArgs) : 1];
    fill_ptrs(tup, ptrs, std::index_sequence_for<KArgs...>{});
    return hipLaunchKernel(reinterpret_cast<const void*>(kern), grid, block, ptrs, shmem, s);
}

}  // namespace attn
