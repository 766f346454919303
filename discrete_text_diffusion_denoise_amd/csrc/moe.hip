// Mixture-of-experts half of a layer on gfx950: top-k routing, stable token
// permutation by expert, grouped SwiGLU expert GEMMs and the gated combine.
//
// Report-summary page (animattoys.com), section 2: 128 experts, the 8 best
// suited run for each token; section 5: a 256-token canvas touches many
// distinct experts, so the layer is bound by loading expert weights.  The
// grouped GEMMs therefore stream each expert's weights exactly once per
// group of 64 routed tokens, straight from HBM into MFMA operands, while the
// (small, reused) token rows come through the caches.
#include "common.h"
#include "kernels.h"

namespace dg {

namespace {

__device__ __forceinline__ uint32_t orderable(float z) {
    uint32_t u = __float_as_uint(z);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One wave per token: k rounds of a wave-wide max over (logit, -index).
__global__ __launch_bounds__(256) void route_kernel(MoeArgs a) {
    const int lane = threadIdx.x & 63;
    const long t = (long)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= a.T) return;
    const float* z = a.z + t * a.E;
    uint64_t key[4];
    float zv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int e = lane + 64 * i;
        zv[i] = e < a.E ? z[e] : 0.f;
        key[i] = e < a.E ? ((uint64_t)orderable(zv[i]) << 32) | (uint32_t)(0xFFFFFFFFu - e) : 0;
    }
    float myz = 0.f;   // lane j keeps the j-th selected logit and expert
    int mye = 0;
    for (int j = 0; j < a.k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < 4; ++i) best = key[i] > best ? key[i] : best;
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) {
            uint32_t lo = __shfl_xor((uint32_t)best, o, 64);
            uint32_t hi = __shfl_xor((uint32_t)(best >> 32), o, 64);
            uint64_t other = ((uint64_t)hi << 32) | lo;
            best = other > best ? other : best;
        }
        const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (lane + 64 * i == e) key[i] = 0;
        if (lane == j) {
            myz = z[e];
            mye = e;
        }
    }
    // gates = softmax over the selected logits (selection order)
    const float z0 = __shfl(myz, 0, 64);
    const float ex = lane < a.k ? expf(myz - z0) : 0.f;
    const float s = wave_sum(ex);
    if (lane < a.k) {
        a.route[t * a.k + lane] = mye;
        a.gates[t * a.k + lane] = ex / s;
    }
}

// counts[e] = number of (token, slot) pairs routed to e.
__global__ __launch_bounds__(256) void count_kernel(MoeArgs a) {
    const int e = blockIdx.x;
    const long total = (long)a.T * a.k;
    int c = 0;
    for (long i = threadIdx.x; i < total; i += 256) c += a.route[i] == e;
    __shared__ int part[256];
    part[threadIdx.x] = c;
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) part[threadIdx.x] += part[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) a.counts[e] = part[0];
}

// One wave per expert: exclusive prefix of counts, then a stable, ordered
// placement of the pairs routed to e (ballot + popcount), so the permutation
// is deterministic.
__global__ __launch_bounds__(64) void place_kernel(MoeArgs a) {
    const int e = blockIdx.x, lane = threadIdx.x;
    int off = 0;
    for (int i = lane; i < e; i += 64) off += a.counts[i];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) off += __shfl_xor(off, o, 64);
    if (lane == 0) {
        a.offsets[e] = off;
        if (e == a.E - 1) a.offsets[a.E] = off + a.counts[e];
    }
    const long total = (long)a.T * a.k;
    const uint64_t lt = (lane == 0) ? 0ull : ((~0ull) >> (64 - lane));
    int run = off;
    for (long base = 0; base < total; base += 64) {
        const long i = base + lane;
        const bool match = i < total && a.route[i] == e;
        const uint64_t mask = __ballot(match);
        if (match) {
            const int slot = run + __popcll(mask & lt);
            a.perm_tok[slot] = (int32_t)(i / a.k);
            a.slot_of[i] = slot;
        }
        run += __popcll(mask);
    }
}

constexpr int MT = 4;     // 16-row token tiles per group (64 routed tokens)
constexpr int KB = 128;   // K elements per lane-contiguous block (4 fragments of 8)

// act[slot][f] = silu(u W_gate^T)[f] * (u W_up^T)[f] for the tokens of expert
// blockIdx.y, f in a 64-wide block.  Wave w owns 16 f-columns; lane (g4, r16)
// streams 32 consecutive k of weight row f0 + r16 per block (the same 32 k of
// each token row), so every weight byte is read once per token group.
template <typename T>
__global__ __launch_bounds__(256) void gateup_kernel(MoeArgs a) {
    const int e = blockIdx.y;
    const int off = a.offsets[e], cnt = a.offsets[e + 1] - off;
    if (cnt == 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int f = blockIdx.x * 64 + wave * 16 + r16;
    const bool fvalid = f < a.F;
    const T* Wg = reinterpret_cast<const T*>(a.w_gate) + ((long)e * a.F + (fvalid ? f : 0)) * a.d;
    const T* Wu = reinterpret_cast<const T*>(a.w_up) + ((long)e * a.F + (fvalid ? f : 0)) * a.d;
    const T* U = reinterpret_cast<const T*>(a.u);
    T* act = reinterpret_cast<T*>(a.act);

    for (int mg = 0; mg < cnt; mg += 16 * MT) {
        long tok[MT];
        bool tv[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int row = mg + 16 * mt + r16;
            tv[mt] = row < cnt;
            tok[mt] = tv[mt] ? a.perm_tok[off + row] : 0;
        }
        f32x4_t ag[MT], au[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            ag[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            au[mt] = ag[mt];
        }
        for (int k0 = 0; k0 < a.d; k0 += KB) {
            Frag<T> bg[4], bu[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k = k0 + g4 * 32 + s * 8;
                if (fvalid && k < a.d) {
                    load_frag(bg[s], Wg + k);
                    load_frag(bu[s], Wu + k);
                } else {
                    zero_frag(bg[s]);
                    zero_frag(bu[s]);
                }
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mg + 16 * mt >= cnt) break;   // uniform across the wave
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int k = k0 + g4 * 32 + s * 8;
                    Frag<T> fa;
                    if (tv[mt] && k < a.d) load_frag(fa, U + tok[mt] * a.d + k);
                    else zero_frag(fa);
                    mma(ag[mt], fa, bg[s]);
                    mma(au[mt], fa, bu[s]);
                }
            }
        }
        if (!fvalid) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = mg + 16 * mt + 4 * g4 + i;
                if (row >= cnt) continue;
                const float gv = ag[mt][i], uv = au[mt][i];
                const float sv = gv / (1.0f + __expf(-gv));
                act[(long)(off + row) * a.F + f] = Elt<T>::from_f(sv * uv);
            }
    }
}

// y[slot][c] = act[slot] . W_down[e][c] for a 64-wide block of output
// columns c (fp32 out).
template <typename T>
__global__ __launch_bounds__(256) void down_kernel(MoeArgs a) {
    const int e = blockIdx.y;
    const int off = a.offsets[e], cnt = a.offsets[e + 1] - off;
    if (cnt == 0) return;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int r16 = lane & 15, g4 = lane >> 4;
    const int c = blockIdx.x * 64 + wave * 16 + r16;
    const bool cvalid = c < a.d;
    const T* Wd = reinterpret_cast<const T*>(a.w_down) + ((long)e * a.d + (cvalid ? c : 0)) * a.F;
    const T* act = reinterpret_cast<const T*>(a.act);

    for (int mg = 0; mg < cnt; mg += 16 * MT) {
        f32x4_t acc[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        for (int k0 = 0; k0 < a.F; k0 += KB) {
            Frag<T> bw[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const int k = k0 + g4 * 32 + s * 8;
                if (cvalid && k < a.F) load_frag(bw[s], Wd + k);
                else zero_frag(bw[s]);
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                if (mg + 16 * mt >= cnt) break;
                const int row = mg + 16 * mt + r16;
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    const int k = k0 + g4 * 32 + s * 8;
                    Frag<T> fa;
                    if (row < cnt && k < a.F) load_frag(fa, act + (long)(off + row) * a.F + k);
                    else zero_frag(fa);
                    mma(acc[mt], fa, bw[s]);
                }
            }
        }
        if (!cvalid) continue;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int row = mg + 16 * mt + 4 * g4 + i;
                if (row < cnt) a.y[(long)(off + row) * a.d + c] = acc[mt][i];
            }
    }
}

// h[t] += sum_j gate[t][j] * y[slot_of[t][j]]  (j in selection order)
__global__ __launch_bounds__(256) void combine_kernel(MoeArgs a) {
    const long t = blockIdx.x;
    for (int c = threadIdx.x; c < a.d; c += 256) {
        float acc = a.h[t * a.d + c];
        for (int j = 0; j < a.k; ++j)
            acc += a.gates[t * a.k + j] * a.y[(long)a.slot_of[t * a.k + j] * a.d + c];
        a.h[t * a.d + c] = acc;
    }
}

}  // namespace

hipError_t moe_route(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    hipLaunchKernelGGL(route_kernel, dim3(cdiv(a.T, 4)), dim3(256), 0, st, a);
    hipLaunchKernelGGL(count_kernel, dim3(a.E), dim3(256), 0, st, a);
    hipLaunchKernelGGL(place_kernel, dim3(a.E), dim3(64), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t moe_gateup(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    hipLaunchKernelGGL(gateup_kernel<T>, dim3(cdiv(a.F, 64), a.E), dim3(256), 0, st, a);
    return hipGetLastError();
}

template <typename T>
hipError_t moe_down(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    hipLaunchKernelGGL(down_kernel<T>, dim3(cdiv(a.d, 64), a.E), dim3(256), 0, st, a);
    return hipGetLastError();
}

hipError_t moe_combine(const MoeArgs& a, hipStream_t st) {
    if (a.T <= 0) return hipSuccess;
    hipLaunchKernelGGL(combine_kernel, dim3(a.T), dim3(256), 0, st, a);
    return hipGetLastError();
}

template hipError_t moe_gateup<bf16_t>(const MoeArgs&, hipStream_t);
template hipError_t moe_gateup<float>(const MoeArgs&, hipStream_t);
template hipError_t moe_down<bf16_t>(const MoeArgs&, hipStream_t);
template hipError_t moe_down<float>(const MoeArgs&, hipStream_t);

}  // namespace dg
