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

#include <utility>

#include "device_common.h"
#include "launch.h"

namespace ttt {
namespace {

// n consecutive elements starting at p (aligned to their total size, up to 16
// bytes), widened to fp32.
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
__device__ __forceinline__ void load_row(const uint16_t* p, float (&out)[N])
{
    // N bf16 values = N/2 dwords
    if constexpr (N >= 8) {
#pragma unroll
        for (int i = 0; i < N; i += 8) {
            const uint4 v = *reinterpret_cast<const uint4*>(p + i);
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                out[i + 2 * j] = __uint_as_float(w[j] << 16);
                out[i + 2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
            }
        }
    } else if constexpr (N == 4) {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        out[0] = __uint_as_float(v.x << 16); out[1] = __uint_as_float(v.x & 0xffff0000u);
        out[2] = __uint_as_float(v.y << 16); out[3] = __uint_as_float(v.y & 0xffff0000u);
    } else if constexpr (N == 2) {
        const uint32_t v = *reinterpret_cast<const uint32_t*>(p);
        out[0] = __uint_as_float(v << 16); out[1] = __uint_as_float(v & 0xffff0000u);
    } else {
        out[0] = bf16_bits_to_f32(*p);
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

// Sum over the 16 lanes of a DPP row (lanes 16m .. 16m+15); every lane of the row
// receives the sum.  Swaps inside each quad (lane ^ 1, lane ^ 2), then the
// half-row mirror (quad 0 <-> quad 1 of each 8-lane half) and the row mirror
// (half 0 <-> half 1); no cross-row movement, no LDS.
__device__ __forceinline__ float dpp_add(float x, int y)
{
    return x + __int_as_float(y);
}

__device__ __forceinline__ float row_sum16(float x)
{
    constexpr int kQuadXor1 = 0xB1;     // quad_perm [1, 0, 3, 2]
    constexpr int kQuadXor2 = 0x4E;     // quad_perm [2, 3, 0, 1]
    constexpr int kRowHalfMirror = 0x141;
    constexpr int kRowMirror = 0x140;
    x = dpp_add(x, __builtin_amdgcn_mov_dpp(__float_as_int(x), kQuadXor1, 0xF, 0xF, false));
    x = dpp_add(x, __builtin_amdgcn_mov_dpp(__float_as_int(x), kQuadXor2, 0xF, 0xF, false));
    x = dpp_add(x, __builtin_amdgcn_mov_dpp(__float_as_int(x), kRowHalfMirror, 0xF, 0xF, false));
    x = dpp_add(x, __builtin_amdgcn_mov_dpp(__float_as_int(x), kRowMirror, 0xF, 0xF, false));
    return x;
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
template <typename TIO, int D>
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

    // inputs of the next kPrefetch tokens in a register ring (token t in slot
    // t % kPrefetch; nothing is loaded past the last token)
    float kr[kPrefetch][C], qr[kPrefetch][C], vr[kPrefetch], er[kPrefetch];
    auto load = [&](int t, auto slot) {
        constexpr int j = decltype(slot)::value;
        if (t >= n) return;
        const size_t tok = tok0 + t;
        load_row(K + tok * D + cg * C, kr[j]);
        load_row(Q + tok * D + cg * C, qr[j]);
        vr[j] = io<TIO>::load(V, tok * D + row);
        er[j] = eta ? eta[tok] : eta_scalar;
    };
    static_for<kPrefetch>([&](auto j) { load(decltype(j)::value, j); });

    int p = pos;
    bool folded = false;
    for (int t0 = 0; t0 < n; t0 += kPrefetch) {
        static_for<kPrefetch>([&](auto slot) {
            constexpr int j = decltype(slot)::value;
            const int t = t0 + j;
            if (t >= n) return;
            float k[C], q[C];
#pragma unroll
            for (int i = 0; i < C; ++i) {
                k[i] = kr[j][i];
                q[i] = qr[j][i];
            }
            const float v = vr[j], et = er[j];
            load(t + kPrefetch, slot);
            // e = W_c k - v
            float s = 0.f;
#pragma unroll
            for (int i = 0; i < C; ++i) s = fmaf(ws[i], k[i], s);
            const float e = row_sum16(s) - v;
            // G += eta e k^T;  z = (W_c - G) q
            float zs = 0.f;
#pragma unroll
            for (int i = 0; i < C; ++i) {
                gg[i] = fmaf(et * e, k[i], gg[i]);
                zs = fmaf(ws[i] - gg[i], q[i], zs);
            }
            const float z = row_sum16(zs);
            if (cg == 0) io<TIO>::store(Z, (tok0 + t) * D + row, z);
            // chunk complete: the updated state becomes the next chunk-start state
            if (++p == chunk) {
                p = 0;
                folded = true;
#pragma unroll
                for (int i = 0; i < C; ++i) {
                    ws[i] -= gg[i];
                    gg[i] = 0.f;
                }
            }
        });
    }

    // the chunk-start state changes only when a chunk completed in this call
    if (folded) store_row(w, ws);
    store_row(gp, gg);
}

template <typename TIO>
hipError_t launch_typed(const LinearArgs& a, float* G, int pos, hipStream_t s)
{
    dim3 grid((unsigned)(a.BH * (a.d / 16))), block(256);
    const TIO* K = (const TIO*)a.K;
    const TIO* Q = (const TIO*)a.Q;
    const TIO* V = (const TIO*)a.V;
    TIO* Z = (TIO*)a.Z;
    // the state is updated in place: W_out is the carried chunk-start state
    switch (a.d) {
    case 16:
        hipLaunchKernelGGL((linear_step_kernel<TIO, 16>), grid, block, 0, s, K, Q, V, a.eta,
                           a.eta_scalar, a.W_out, G, Z, a.T, a.chunk, pos);
        break;
    case 32:
        hipLaunchKernelGGL((linear_step_kernel<TIO, 32>), grid, block, 0, s, K, Q, V, a.eta,
                           a.eta_scalar, a.W_out, G, Z, a.T, a.chunk, pos);
        break;
    case 64:
        hipLaunchKernelGGL((linear_step_kernel<TIO, 64>), grid, block, 0, s, K, Q, V, a.eta,
                           a.eta_scalar, a.W_out, G, Z, a.T, a.chunk, pos);
        break;
    case 128:
        hipLaunchKernelGGL((linear_step_kernel<TIO, 128>), grid, block, 0, s, K, Q, V, a.eta,
                           a.eta_scalar, a.W_out, G, Z, a.T, a.chunk, pos);
        break;
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
