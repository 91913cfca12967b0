// HBM-streaming kernels of the Muon step: momentum + bf16 cast, the Frobenius
// normaliser, and the float32 apply with decoupled weight decay.
//
// Each is bound by HBM bandwidth, not arithmetic: per element the momentum kernel moves
// 14 bytes (fp32 G) or 12 (bf16 G), the apply kernel 10, the normaliser 4.  Work is cut
// into 64 x 64 tiles of the parameter's own rows x cols; every access to W, M and G is a
// 16-byte vector per lane along the contiguous dimension.  A matrix stored canonically
// as its transpose (rows > cols) goes through a 64 x 64 LDS tile so that both the read
// of the parameter and the write of X (or the read of O) stay coalesced.
//
// Bitwise agreement with the float64 oracle: the momentum and apply arithmetic is done
// in float64 with each product and sum rounded as written (contraction is off in this
// file), then rounded once to float32; bf16 casts round to nearest even.
#include "device_common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace muon {
namespace {

using dev::bf16_to_f32;
using dev::f32_to_bf16;
using dev::f64_to_bf16;

constexpr int T = EW_TILE;      // 64
constexpr int LDT = T + 8;      // LDS row stride (bf16) of a transpose tile: 144 B

// ---------------------------------------------------------------------------------------
// Step 1 of the pages' optimizer step: M <- beta*M + (1-beta)*G in FP32, X0 = bf16(M).
// ---------------------------------------------------------------------------------------
template <int GDT>
__device__ __forceinline__ void load_grad4(const void* g, int64_t idx, float out[4]) {
    if (GDT == MUON_DTYPE_F32) {
        const float4 v = *reinterpret_cast<const float4*>(static_cast<const float*>(g) + idx);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g) + idx);
        out[0] = bf16_to_f32(v.x & 0xffffu); out[1] = bf16_to_f32(v.x >> 16);
        out[2] = bf16_to_f32(v.y & 0xffffu); out[3] = bf16_to_f32(v.y >> 16);
    }
}

template <int GDT>
__device__ __forceinline__ float load_grad1(const void* g, int64_t idx) {
    if (GDT == MUON_DTYPE_F32) return static_cast<const float*>(g)[idx];
    return bf16_to_f32(static_cast<const uint16_t*>(g)[idx]);
}

__device__ __forceinline__ float momentum_elem(float m, float g, double beta, double omb) {
    const double p1 = beta * (double)m;   // exact: 24 x 24 significant bits
    const double p2 = omb * (double)g;    // exact
    return (float)(p1 + p2);              // one float64 rounding, then one float32 rounding
}

template <int GDT>
__global__ __launch_bounds__(256) void momentum_kernel(MomentumArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t tr[T][LDT];
    __shared__ double red[4];
    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;
    const double beta = (double)a.beta, omb = (double)a.omb;

    for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int64_t mat = t / a.ew_tiles;
        const int64_t tile = t - mat * a.ew_tiles;
        const MatEntry e = a.tbl[mat];
        const int64_t tiles_c = (e.cols + T - 1) / T;
        const int64_t r0 = (tile / tiles_c) * T, c0 = (tile % tiles_c) * T;
        const bool vec = (e.cols & 3) == 0;
        uint16_t* X = a.xq + mat * a.mat_stride;
        const int64_t c = c0 + cg * 4;
        double ss = 0.0;

#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = r0 + rg + 16 * i;
            uint16_t xb[4] = {0, 0, 0, 0};
            int nvalid = 0;
            if (r < e.rows && c < e.cols) {
                const int64_t base = r * e.cols + c;
                if (vec && c + 4 <= e.cols) {
                    nvalid = 4;
                    const float4 mv = *reinterpret_cast<const float4*>(e.m + base);
                    float gv[4];
                    load_grad4<GDT>(e.g, base, gv);
                    float4 mn;
                    mn.x = momentum_elem(mv.x, gv[0], beta, omb);
                    mn.y = momentum_elem(mv.y, gv[1], beta, omb);
                    mn.z = momentum_elem(mv.z, gv[2], beta, omb);
                    mn.w = momentum_elem(mv.w, gv[3], beta, omb);
                    *reinterpret_cast<float4*>(e.m + base) = mn;
                    xb[0] = f32_to_bf16(mn.x); xb[1] = f32_to_bf16(mn.y);
                    xb[2] = f32_to_bf16(mn.z); xb[3] = f32_to_bf16(mn.w);
                } else {
                    nvalid = (int)((e.cols - c) < 4 ? (e.cols - c) : 4);
                    for (int j = 0; j < nvalid; ++j) {
                        const float mn = momentum_elem(e.m[base + j], load_grad1<GDT>(e.g, base + j), beta, omb);
                        e.m[base + j] = mn;
                        xb[j] = f32_to_bf16(mn);
                    }
                }
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const double x = (double)bf16_to_f32(xb[j]);
                    ss += x * x;    // exact square (8-bit significand); sum in float64
                }
            }
            if (!e.trans) {
                if (nvalid == 4 && ((a.np & 3) == 0)) {
                    uint2 v;
                    v.x = (uint32_t)xb[0] | ((uint32_t)xb[1] << 16);
                    v.y = (uint32_t)xb[2] | ((uint32_t)xb[3] << 16);
                    *reinterpret_cast<uint2*>(X + r * a.np + c) = v;
                } else {
                    for (int j = 0; j < nvalid; ++j) X[r * a.np + c + j] = xb[j];
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) tr[cg * 4 + j][rg + 16 * i] = xb[j];
            }
        }

        if (e.trans) {
            // X0 = M^T: row q of X0 is column c0 + q of M; its columns are M's rows.
            __syncthreads();
            const int q = tid >> 2, seg = (tid & 3) * 16;
            const int64_t xr = c0 + q;
            const int64_t xc = r0 + seg;
            if (xr < e.cols && xc < e.rows) {
                uint16_t* dst = X + xr * a.np + xc;
                if (xc + 16 <= e.rows) {
                    const uint4* srcv = reinterpret_cast<const uint4*>(&tr[q][seg]);
                    reinterpret_cast<uint4*>(dst)[0] = srcv[0];
                    reinterpret_cast<uint4*>(dst)[1] = srcv[1];
                } else {
                    for (int k = 0; xc + k < e.rows; ++k) dst[k] = tr[q][seg + k];
                }
            }
        }

        // block sum of squares in a fixed order -> this tile's partial
        ss = dev::wave_sum(ss);
        if ((tid & 63) == 0) red[tid >> 6] = ss;
        __syncthreads();
        if (tid == 0) a.partials[t] = (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------
// Normaliser: inv = 1 / (sqrt(sum of squares) + eps) per matrix, then X = bf16(X0 * inv).
// ---------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs a) {
    __shared__ double red[4];
    const int tid = threadIdx.x;
    const int64_t mat = blockIdx.x;
    const double* p = a.partials + mat * a.ew_tiles;
    double s = 0.0;
    for (int64_t i = tid; i < a.ew_tiles; i += 256) s += p[i];
    s = dev::wave_sum(s);
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __syncthreads();
    if (tid == 0) {
        const double tot = (red[0] + red[1]) + (red[2] + red[3]);
        a.inv[mat] = 1.0 / (sqrt(tot) + a.eps);
    }
}

__global__ __launch_bounds__(256) void normalize_kernel(NormalizeArgs a) {
    const int64_t upr = a.np >> 3;             // 8-element units per row
    const int64_t per_mat = a.mp * upr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < a.total_units; u += stride) {
        const int64_t mat = u / per_mat;
        const int64_t rem = u - mat * per_mat;
        const int64_t r = rem / upr;
        const int64_t c = (rem - r * upr) * 8;
        const int64_t off = mat * a.mp * a.np + r * a.np + c;
        uint4 out = make_uint4(0, 0, 0, 0);
        if (r < a.m && c < a.n) {
            const double s = a.inv[mat];
            const uint4 in = *reinterpret_cast<const uint4*>(a.src + off);
            const uint32_t w[4] = {in.x, in.y, in.z, in.w};
            uint32_t o[4] = {0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (c + j < a.n) {
                    const uint32_t h = (j & 1) ? (w[j >> 1] >> 16) : (w[j >> 1] & 0xffffu);
                    const uint32_t y = f64_to_bf16((double)bf16_to_f32(h) * s);
                    o[j >> 1] |= (j & 1) ? (y << 16) : y;
                }
            }
            out = make_uint4(o[0], o[1], o[2], o[3]);
        }
        *reinterpret_cast<uint4*>(a.dst + off) = out;
    }
}

// ---------------------------------------------------------------------------------------
// Step 5: W <- f32(d*W - u*O), d = 1 - lr*wd, u = lr*s_i, each operation one float64
// rounding (contraction is off in this file).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ float apply_elem(float w, float o, double d, double u) {
    const double t1 = d * (double)w;
    const double t2 = u * (double)o;
    return (float)(t1 - t2);
}

__global__ __launch_bounds__(256) void apply_kernel(ApplyArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t tr[T][LDT];
    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;

    for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int64_t mat = t / a.ew_tiles;
        const int64_t tile = t - mat * a.ew_tiles;
        const MatEntry e = a.tbl[mat];
        const int64_t tiles_c = (e.cols + T - 1) / T;
        const int64_t r0 = (tile / tiles_c) * T, c0 = (tile % tiles_c) * T;
        const bool vec = (e.cols & 3) == 0;
        const uint16_t* O = a.xo + mat * a.mat_stride;
        const double u = (double)a.lr * (double)e.scale;   // exact
        const int64_t c = c0 + cg * 4;

        if (e.trans) {
            // O is stored as the cols x rows transpose: stage O^T's 64 x 64 block in LDS.
            const int q = tid >> 2, seg = (tid & 3) * 16;
            const int64_t orow = c0 + q;       // canonical row = parameter column
            const int64_t ocol = r0 + seg;     // canonical column = parameter row
            if (orow < e.cols && ocol < e.rows) {
                const uint16_t* src = O + orow * a.np + ocol;
                if (ocol + 16 <= e.rows) {
                    uint4* d4 = reinterpret_cast<uint4*>(&tr[q][seg]);
                    d4[0] = reinterpret_cast<const uint4*>(src)[0];
                    d4[1] = reinterpret_cast<const uint4*>(src)[1];
                } else {
                    for (int k = 0; ocol + k < e.rows; ++k) tr[q][seg + k] = src[k];
                }
            }
            __syncthreads();
        }

#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int64_t r = r0 + rg + 16 * i;
            if (r >= e.rows || c >= e.cols) continue;
            const int64_t base = r * e.cols + c;
            const int nvalid = (int)((e.cols - c) < 4 ? (e.cols - c) : 4);
            float o[4] = {0.f, 0.f, 0.f, 0.f};
            if (e.trans) {
                for (int j = 0; j < nvalid; ++j) o[j] = bf16_to_f32(tr[cg * 4 + j][rg + 16 * i]);
            } else if (nvalid == 4 && (a.np & 3) == 0) {
                const uint2 v = *reinterpret_cast<const uint2*>(O + r * a.np + c);
                o[0] = bf16_to_f32(v.x & 0xffffu); o[1] = bf16_to_f32(v.x >> 16);
                o[2] = bf16_to_f32(v.y & 0xffffu); o[3] = bf16_to_f32(v.y >> 16);
            } else {
                for (int j = 0; j < nvalid; ++j) o[j] = bf16_to_f32(O[r * a.np + c + j]);
            }
            if (vec && nvalid == 4) {
                float4 w = *reinterpret_cast<const float4*>(e.w + base);
                w.x = apply_elem(w.x, o[0], a.d, u);
                w.y = apply_elem(w.y, o[1], a.d, u);
                w.z = apply_elem(w.z, o[2], a.d, u);
                w.w = apply_elem(w.w, o[3], a.d, u);
                *reinterpret_cast<float4*>(e.w + base) = w;
            } else {
                for (int j = 0; j < nvalid; ++j) e.w[base + j] = apply_elem(e.w[base + j], o[j], a.d, u);
            }
        }
        if (e.trans) __syncthreads();
    }
}

// Grid size for the grid-stride loops: enough blocks to fill 256 CUs many times over.
inline unsigned grid_for(int64_t items, int64_t cap = 256 * 64) {
    return (unsigned)(items < cap ? (items > 0 ? items : 1) : cap);
}

}  // namespace

hipError_t launch_momentum(const MomentumArgs& a, int32_t grad_dtype, hipStream_t s) {
    const unsigned grid = grid_for(a.total_tiles);
    if (grad_dtype == MUON_DTYPE_F32)
        hipLaunchKernelGGL(momentum_kernel<MUON_DTYPE_F32>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(momentum_kernel<MUON_DTYPE_BF16>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, int64_t count, hipStream_t s) {
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)count), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_normalize(const NormalizeArgs& a, hipStream_t s) {
    const unsigned grid = grid_for((a.total_units + 255) / 256, 256 * 16);
    hipLaunchKernelGGL(normalize_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_apply(const ApplyArgs& a, hipStream_t s) {
    const unsigned grid = grid_for(a.total_tiles);
    hipLaunchKernelGGL(apply_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace muon
