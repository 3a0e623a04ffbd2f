// Streaming continuation of the TTT-Linear scan (decode): n more tokens of each
// (batch, head) sequence from a carried state.
//
// Within a chunk every gradient is taken at the chunk-start state W_c and token t
// reads the chunk's updates up to and including its own (PaperTrace "5 ·
// TestingTime 训练与长上下文" §1.1, §2.1, §2.3).  The carried state is therefore
// the pair (W_c, G) with G = sum over the chunk's tokens so far of
// eta_s (W_c k_s - v_s) k_s^T, plus the position in the chunk.  Per token:
//     e = W_c k - v,   G += eta e k^T,   z = (W_c - G) q,
// and when a chunk completes, W_c <- W_c - G and G <- 0.
//
// One 256-thread workgroup per (batch*head, 16 state rows): 16 lanes per row,
// each holding d/16 consecutive columns of W_c and G in registers (fp32
// arithmetic, the reductions over a row by DPP moves inside a 16-lane row).  The
// inputs of the next few tokens are in flight while one is processed.
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "device_common.h"
#include "launch.h"

namespace ttt {
namespace {

// n consecutive fp32 elements starting at p (aligned to their total size, up to
// 16 bytes)
template <int N>
__device__ __forceinline__ void load_row(const float* p, float (&out)[N])
{
    if constexpr (N >= 4) {
#pragma unroll
        for (int i = 0; i < N; i += 4) {
            const float4 v = *reinterpret_cast<const float4*>(p + i);
            out[i] = v.x; out[i + 1] = v.y; out[i + 2] = v.z; out[i + 3] = v.w;
        }
    } else if constexpr (N == 2) {
        const float2 v = *reinterpret_cast<const float2*>(p);
        out[0] = v.x; out[1] = v.y;
    } else {
        out[0] = *p;
    }
}

template <int N>
__device__ __forceinline__ void store_row(float* p, const float (&v)[N])
{
    if constexpr (N >= 4) {
#pragma unroll
        for (int i = 0; i < N; i += 4)
            *reinterpret_cast<float4*>(p + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
    } else if constexpr (N == 2) {
        *reinterpret_cast<float2*>(p) = make_float2(v[0], v[1]);
    } else {
        *p = v[0];
    }
}

// f(integral_constant<0>), ..., f(integral_constant<N-1>): ring slots as constants
template <typename F, int... I>
__device__ __forceinline__ void static_for_seq(F& f, std::integer_sequence<int, I...>)
{
    (f(std::integral_constant<int, I>{}), ...);
}

template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_seq(f, std::make_integer_sequence<int, N>{});
}

// tokens whose inputs are in flight ahead of the one being processed
constexpr int kPrefetch = 4;

// Lane (r, cg) of the workgroup holds state row 16*blockIdx + r, columns
// [cg*C, cg*C + C), C = D/16: every state row is read and written as contiguous
// 16-byte pieces and a key/query row as one contiguous segment per row group.
// ETA: per-token learning rates (else eta_scalar for every token).
template <typename TIO, int D, bool ETA>
__global__ __launch_bounds__(256) void linear_step_kernel(
    const TIO* __restrict__ K, const TIO* __restrict__ Q, const TIO* __restrict__ V,
    const float* __restrict__ eta, float eta_scalar, float* __restrict__ Wc,
    float* __restrict__ G, TIO* __restrict__ Z, int n, int chunk, int pos)
{
    constexpr int C = D / 16, NRB = D / 16;
    const int tid = threadIdx.x;
    const int r = tid >> 4, cg = tid & 15;
    const int slice = blockIdx.x / NRB;
    const int row = (blockIdx.x % NRB) * 16 + r;
    const size_t tok0 = (size_t)slice * n;
    float* w = Wc + ((size_t)slice * D + row) * D + cg * C;
    float* gp = G + ((size_t)slice * D + row) * D + cg * C;

    float ws[C], gg[C];
    load_row(w, ws);
    load_row(gp, gg);

    // Inputs of the next kPrefetch tokens in a register ring, token t in slot
    // t % kPrefetch, kept as loaded words.  A slot is refilled right after its
    // token is done.  Every path through the ring issues the same loads (a
    // refill past the last token re-reads the last one), so the wait for a slot
    // covers that slot's loads only, not the later loads and Z stores.
    RawRow<TIO, C> kr[kPrefetch], qr[kPrefetch];
    RawRow<TIO, 1> vr[kPrefetch];
    float er[kPrefetch];
    auto load = [&](int t, auto slot) {
        constexpr int j = decltype(slot)::value;
        const size_t tok = tok0 + t;
        kr[j].load(K + tok * D + cg * C);
        qr[j].load(Q + tok * D + cg * C);
        vr[j].load(V + tok * D + row);
        if constexpr (ETA) er[j] = eta[tok];
        else er[j] = eta_scalar;
    };
    int p = pos;
    bool folded = false;
    auto process = [&](int t, auto slot) {
        constexpr int j = decltype(slot)::value;
        // e = W_c k - v
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < C; ++i) s = fmaf(ws[i], kr[j].at(i), s);
        const float e = row_sum16(s) - vr[j].at(0);
        // G += eta e k^T;  z = (W_c - G) q
        const float ee = er[j] * e;
        float zs = 0.f;
#pragma unroll
        for (int i = 0; i < C; ++i) {
            gg[i] = fmaf(ee, kr[j].at(i), gg[i]);
            zs = fmaf(ws[i] - gg[i], qr[j].at(i), zs);
        }
        const float z = row_sum16(zs);
        if (cg == 0) io<TIO>::store(Z, (tok0 + t) * D + row, z);
    };
    // chunk complete: the updated state becomes the next chunk-start state
    auto advance = [&]() {
        if (++p == chunk) {
            p = 0;
            folded = true;
#pragma unroll
            for (int i = 0; i < C; ++i) {
                ws[i] -= gg[i];
                gg[i] = 0.f;
            }
        }
    };
    // token 0 (n >= 1) is fetched together with the state rows: a one-token
    // call makes one memory round trip
    const std::integral_constant<int, 0> slot0;
    load(0, slot0);
    __builtin_amdgcn_sched_barrier(0);
    if (n >= kPrefetch) {
        // the other slots one by one, in the order the refills repeat (the
        // scheduler would otherwise group the loads by tensor, and the first pass
        // through the ring would then wait for every load of the ring at slot 0)
        static_for<kPrefetch>([&](auto j) {
            if constexpr (decltype(j)::value > 0) {
                load(decltype(j)::value, j);
                __builtin_amdgcn_sched_barrier(0);
            }
        });
        int t0 = 0;
        for (; t0 + kPrefetch <= n; t0 += kPrefetch) {
            static_for<kPrefetch>([&](auto slot) {
                const int t = t0 + decltype(slot)::value;
                process(t, slot);
                load(min(t + kPrefetch, n - 1), slot);
                advance();
            });
        }
        // the last n % kPrefetch tokens are already in slots 0, 1, ...
        static_for<kPrefetch>([&](auto slot) {
            const int t = t0 + decltype(slot)::value;
            if (t < n) {
                process(t, slot);
                advance();
            }
        });
    } else {
        for (int t = 0; t < n; ++t) {
            if (t > 0) load(t, slot0);
            process(t, slot0);
            advance();
        }
    }

    // the chunk-start state changes only when a chunk completed in this call
    if (folded) store_row(w, ws);
    store_row(gp, gg);
}

template <typename TIO, int D>
void launch_d(const LinearArgs& a, float* G, int pos, hipStream_t s)
{
    dim3 grid((unsigned)(a.BH * (D / 16))), block(256);
    const TIO* K = (const TIO*)a.K;
    const TIO* Q = (const TIO*)a.Q;
    const TIO* V = (const TIO*)a.V;
    TIO* Z = (TIO*)a.Z;
    // the state is updated in place: W_out is the carried chunk-start state
    if (a.eta)
        hipLaunchKernelGGL((linear_step_kernel<TIO, D, true>), grid, block, 0, s, K, Q, V, a.eta,
                           a.eta_scalar, a.W_out, G, Z, a.T, a.chunk, pos);
    else
        hipLaunchKernelGGL((linear_step_kernel<TIO, D, false>), grid, block, 0, s, K, Q, V,
                           a.eta, a.eta_scalar, a.W_out, G, Z, a.T, a.chunk, pos);
}

template <typename TIO>
hipError_t launch_typed(const LinearArgs& a, float* G, int pos, hipStream_t s)
{
    switch (a.d) {
    case 16: launch_d<TIO, 16>(a, G, pos, s); break;
    case 32: launch_d<TIO, 32>(a, G, pos, s); break;
    case 64: launch_d<TIO, 64>(a, G, pos, s); break;
    case 128: launch_d<TIO, 128>(a, G, pos, s); break;
    default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_step(const LinearArgs& a, float* G, int pos, hipStream_t s)
{
    return a.bf16 ? launch_typed<uint16_t>(a, G, pos, s) : launch_typed<float>(a, G, pos, s);
}

}  // namespace ttt
