// The query rotation q' = R_k q ("MosaicKV 阅读笔记" reading notes, Eq. 12;
// paper summary section 5.3), shared by the decode's own launch and by the
// combined append-and-decode launch, which runs it beside the append.
#pragma once

#include "device_util.hpp"
#include "mkv_internal.h"

namespace mkv {

constexpr float kRsqrtD = 0.08838834764831845f;  // 1 / sqrt(128)
constexpr float kLog2e = 1.4426950408889634f;

// One 256-thread workgroup: channels 32 cb .. 32 cb + 31 of q' for the G query
// heads of KV head g of one request, with the rotation Rb ([n_kv][2][D][D],
// R_k used). The 8 lanes of channel c sum 16 columns each of R_k[c] . q (one
// round of 16-byte loads per lane) and add up with DPP (quad swaps, then the
// half-row mirror). q_b: the request's queries [Hq][D]. Writes
//   qa[g G + i][c] = q'_c log2(e) / sqrt(D)
//   qs[g][c][i] = max(q'_c, 0) / sqrt(D),  qs[g][c][G + i] = min(q'_c, 0) / sqrt(D)
// (qa, qs: the request's q' of one rotation slot). qsh: the caller's LDS area
// of at least G x D floats.
template <int G>
__device__ __forceinline__ void qrot_block(const float *__restrict__ Rb, const float *__restrict__ q_b, float *qa,
                                           float *qs_all, int g, int cb, float (*qsh)[D]) {
    const int tid = (int)threadIdx.x;
    const int k = tid & 7;
    const int c = cb * 32 + (tid >> 3);
    const float4 *Rr = reinterpret_cast<const float4 *>(Rb + ((size_t)g * 2) * D * D + (size_t)c * D + 16 * k);
    float4 r[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) r[u] = Rr[u];
    for (int i = tid; i < G * D; i += 256) qsh[i / D][i % D] = q_b[(size_t)g * G * D + i];
    __syncthreads();
    float acc[G];
#pragma unroll
    for (int i = 0; i < G; ++i) {
        const float4 *x4 = reinterpret_cast<const float4 *>(&qsh[i][16 * k]);
        float a = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float4 x = x4[u];
            a = fmaf(r[u].x, x.x, a);
            a = fmaf(r[u].y, x.y, a);
            a = fmaf(r[u].z, x.z, a);
            a = fmaf(r[u].w, x.w, a);
        }
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xf, 0xf, false));
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xf, 0xf, false));
        a += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x141, 0xf, 0xf, false));
        acc[i] = a;
    }
    if (k == 0) {
        float *qs = qs_all + ((size_t)g * D + c) * 2 * G;
#pragma unroll
        for (int i = 0; i < G; ++i) {
            qa[(size_t)(g * G + i) * D + c] = acc[i] * (kRsqrtD * kLog2e);
            qs[i] = fmaxf(acc[i], 0.f) * kRsqrtD;
            qs[G + i] = fminf(acc[i], 0.f) * kRsqrtD;
        }
    }
}

}  // namespace mkv
