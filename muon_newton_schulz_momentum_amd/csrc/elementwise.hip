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
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

#pragma clang fp contract(off)

namespace muon {
namespace {

using dev::bf16_to_f32;
using dev::f32_to_bf16;

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

// The bf16 matrix handed to Newton–Schulz: the new momentum itself, or with Nesterov the
// look-ahead beta*M_new + (1-beta)*G, formed exactly like the momentum (float64 products
// and sum, one float32 rounding) and then cast.
__device__ __forceinline__ uint16_t x0_bits(float mn, float g, bool nesterov, double beta, double omb) {
    return f32_to_bf16(nesterov ? momentum_elem(mn, g, beta, omb) : mn);
}

template <int GDT>
__global__ __launch_bounds__(256) void momentum_kernel(MomentumArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t tr[T][LDT];
    __shared__ double red[4];
    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;
    float beta32 = a.beta, omb32 = a.omb;
    if (a.dev_scalars) {            // beta from device memory; (1 - beta) formed as the host forms it
        beta32 = a.dev_scalars[0];
        omb32 = 1.0f - beta32;
    }
    const double beta = (double)beta32, omb = (double)omb32;
    const bool nest = a.nesterov != 0;

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
        // A parameter stored as it is (not transposed) is streamed flat: tile t covers its
        // elements [4096 t, 4096 t + 4096) in row-major order, lane l of a wave handles 16
        // bytes at 1 KB steps, so every wave access is 1 KB contiguous (a 64 x 64 tile
        // would touch 64 separate 256-byte row pieces).  All loads go out before the first
        // store.  The tile's sum of squares lands in its own partial, as in the 2-D path.
        const bool flat = !e.trans && vec && (a.np & 3) == 0;
        if (flat) {
            const int64_t nel = e.rows * e.cols;
            const int64_t e0 = tile * (T * T) + tid * 4;
            float4 mv[4];
            float gv[4][4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t idx = e0 + k * 1024;
                if (idx < nel) {
                    mv[k] = *reinterpret_cast<const float4*>(e.m + idx);
                    load_grad4<GDT>(e.g, idx, gv[k]);
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t idx = e0 + k * 1024;
                if (idx >= nel) continue;
                float4 mn;
                mn.x = momentum_elem(mv[k].x, gv[k][0], beta, omb);
                mn.y = momentum_elem(mv[k].y, gv[k][1], beta, omb);
                mn.z = momentum_elem(mv[k].z, gv[k][2], beta, omb);
                mn.w = momentum_elem(mv[k].w, gv[k][3], beta, omb);
                *reinterpret_cast<float4*>(e.m + idx) = mn;
                const uint16_t xb[4] = {x0_bits(mn.x, gv[k][0], nest, beta, omb), x0_bits(mn.y, gv[k][1], nest, beta, omb),
                                        x0_bits(mn.z, gv[k][2], nest, beta, omb), x0_bits(mn.w, gv[k][3], nest, beta, omb)};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const double x = (double)bf16_to_f32(xb[j]);
                    ss += x * x;
                }
                // the 4 elements share a row (cols is a multiple of 4)
                const int64_t xi = (a.np == e.cols) ? idx : (idx / e.cols) * a.np + idx % e.cols;
                uint2 v;
                v.x = (uint32_t)xb[0] | ((uint32_t)xb[1] << 16);
                v.y = (uint32_t)xb[2] | ((uint32_t)xb[3] << 16);
                *reinterpret_cast<uint2*>(X + xi) = v;
            }
        }
        // Interior tile: every load of the tile is issued before the first store, so each
        // lane keeps 8 loads in flight (stores to M may alias later loads of M as far as
        // the compiler knows, so the general loop below cannot be reordered that way).
        const bool full = !flat && vec && r0 + T <= e.rows && c0 + T <= e.cols && (a.np & 3) == 0;
        if (full) {
            float4 mv[4];
            float gv[4][4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t base = (r0 + rg + 16 * i) * e.cols + c;
                mv[i] = *reinterpret_cast<const float4*>(e.m + base);
                load_grad4<GDT>(e.g, base, gv[i]);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = r0 + rg + 16 * i;
                const int64_t base = r * e.cols + c;
                float4 mn;
                mn.x = momentum_elem(mv[i].x, gv[i][0], beta, omb);
                mn.y = momentum_elem(mv[i].y, gv[i][1], beta, omb);
                mn.z = momentum_elem(mv[i].z, gv[i][2], beta, omb);
                mn.w = momentum_elem(mv[i].w, gv[i][3], beta, omb);
                *reinterpret_cast<float4*>(e.m + base) = mn;
                const uint16_t xb[4] = {x0_bits(mn.x, gv[i][0], nest, beta, omb), x0_bits(mn.y, gv[i][1], nest, beta, omb),
                                        x0_bits(mn.z, gv[i][2], nest, beta, omb), x0_bits(mn.w, gv[i][3], nest, beta, omb)};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const double x = (double)bf16_to_f32(xb[j]);
                    ss += x * x;
                }
                if (!e.trans) {
                    uint2 v;
                    v.x = (uint32_t)xb[0] | ((uint32_t)xb[1] << 16);
                    v.y = (uint32_t)xb[2] | ((uint32_t)xb[3] << 16);
                    *reinterpret_cast<uint2*>(X + r * a.np + c) = v;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) tr[cg * 4 + j][rg + 16 * i] = xb[j];
                }
            }
        }

#pragma unroll
        for (int i = 0; i < 4 && !full && !flat; ++i) {
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
                    xb[0] = x0_bits(mn.x, gv[0], nest, beta, omb); xb[1] = x0_bits(mn.y, gv[1], nest, beta, omb);
                    xb[2] = x0_bits(mn.z, gv[2], nest, beta, omb); xb[3] = x0_bits(mn.w, gv[3], nest, beta, omb);
                } else {
                    nvalid = (int)((e.cols - c) < 4 ? (e.cols - c) : 4);
                    for (int j = 0; j < nvalid; ++j) {
                        const float gj = load_grad1<GDT>(e.g, base + j);
                        const float mn = momentum_elem(e.m[base + j], gj, beta, omb);
                        e.m[base + j] = mn;
                        xb[j] = x0_bits(mn, gj, nest, beta, omb);
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
// Normaliser: inv = 1 / (sqrt(sum of squares) + eps) per matrix, then X = bf16(X0 * inv)
// (one rounding, through the matrix's float32 scale).
// ---------------------------------------------------------------------------------------
// One matrix's normalisation scale by a 256-thread block: inv = 1 / (sqrt(sum of its tile
// partials) + eps), the partials summed in a fixed order (thread i adds partials i, i + 256,
// ...; each wave's butterfly; then the four waves pairwise), and the float32 scale
// dev::exact_scale(inv) found by the first wave.  Every thread gets the scale, as a double
// (red: 5 doubles of LDS).
__device__ __forceinline__ double block_inv(const double* part, int64_t ew_tiles, double eps, double* red) {
    const int tid = threadIdx.x;
    double s = 0.0;
    for (int64_t i = tid; i < ew_tiles; i += 256) s += part[i];
    s = dev::wave_sum(s);
    if ((tid & 63) == 0) red[tid >> 6] = s;
    __syncthreads();
    if (tid < 64) {
        const double tot = (red[0] + red[1]) + (red[2] + red[3]);
        const float scale = dev::exact_scale(1.0 / (sqrt(tot) + eps));
        if (tid == 0) red[4] = (double)scale;
    }
    __syncthreads();
    return red[4];
}

__global__ __launch_bounds__(256) void finalize_kernel(FinalizeArgs a) {
    __shared__ double red[5];
    const int tid = threadIdx.x;
    if (blockIdx.x == 0 && tid < SCHED_WORDS) a.sched[tid] = 0u;
    const int64_t mat = blockIdx.x;
    const double inv = block_inv(a.partials + mat * a.ew_tiles, a.ew_tiles, a.eps, red);
    if (tid == 0) a.inv[mat] = inv;
    if (a.x0) {
        // X0's padding: the rows past m whole, and columns n .. np-1 of the first m rows
        // (whole 16-byte units from the first multiple of 8 at or past n, single elements
        // before it)
        uint16_t* x = a.x0 + mat * a.mp * a.np;
        const int64_t upr = a.np / 8;                       // 16-byte units per row
        const int64_t c8 = (a.n + 7) / 8;                   // first unit wholly past n
        const int64_t tail = c8 * 8 - a.n;                  // single elements before it
        const int64_t n_rows = (a.mp - a.m) * upr, n_cols = a.m * (upr - c8), n_tail = a.m * tail;
        const uint4 z = make_uint4(0, 0, 0, 0);
        for (int64_t u = tid; u < n_rows; u += 256)
            *reinterpret_cast<uint4*>(x + a.m * a.np + u * 8) = z;
        for (int64_t u = tid; u < n_cols; u += 256) {
            const int64_t r = u / (upr - c8), k = u - r * (upr - c8);
            *reinterpret_cast<uint4*>(x + r * a.np + (c8 + k) * 8) = z;
        }
        for (int64_t u = tid; u < n_tail; u += 256) {
            const int64_t r = u / tail, k = u - r * tail;
            x[r * a.np + a.n + k] = 0;
        }
    }
}

__device__ __forceinline__ uint4 normalize_unit(uint4 in, int64_t c, int64_t n, double s) {
    return dev::normalize8(in, (int32_t)(n - c < 8 ? n - c : 8), (float)s);
}

// The chunk's matrices are mp x np blocks one after another, so unit u (8 elements) is in
// global row R = u / (np / 8) at element offset R * np + 8 * (u mod np / 8), and its matrix
// is R / mp.  Per workgroup pass the base unit's row is found once (uniform, 64-bit); each
// thread then divides only small 32-bit offsets.  (Two 64-bit divisions per unit made the
// kernel bound by vector-ALU work rather than by HBM.)
struct UnitPos {
    int64_t off;      // element offset of the unit in the chunk's X buffers
    int64_t mat;
    bool live;        // inside the matrix's m x n region
    uint32_t c;       // column of the unit's first element
};

__device__ __forceinline__ UnitPos unit_pos(const NormalizeArgs& a, int64_t r0, uint32_t k0, uint32_t d,
                                            uint32_t upr) {
    const uint32_t t = k0 + d;
    const uint32_t q = t / upr;
    const uint32_t k = t - q * upr;
    const int64_t R = r0 + q;
    const uint32_t mp = (uint32_t)a.mp;
    const uint32_t Rm = (uint32_t)R;                  // a chunk has fewer than 2^31 rows (checked at bind)
    const uint32_t mat = Rm / mp;
    const uint32_t r = Rm - mat * mp;
    UnitPos u;
    u.c = k * 8u;
    u.off = R * a.np + u.c;
    u.mat = mat;
    u.live = r < (uint32_t)a.m && u.c < (uint32_t)a.n;
    return u;
}

// Each thread takes UPT units of 8 elements, one block-width apart, and issues all its
// loads before the first store.
constexpr int UPT = 4;

__global__ __launch_bounds__(256) void normalize_kernel(NormalizeArgs a) {
    const uint32_t upr = (uint32_t)(a.np >> 3);          // 8-element units per row
    const int64_t span = (int64_t)gridDim.x * blockDim.x * UPT;
    for (int64_t ub = (int64_t)blockIdx.x * blockDim.x * UPT; ub < a.total_units; ub += span) {
        const int64_t r0 = ub / upr;                      // uniform
        const uint32_t k0 = (uint32_t)(ub - r0 * upr);
        uint4 in[UPT];
        UnitPos pos[UPT];
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            const uint32_t d = threadIdx.x + (uint32_t)k * blockDim.x;
            pos[k] = unit_pos(a, r0, k0, d, upr);
            const bool ok = ub + d < a.total_units && pos[k].live;
            in[k] = ok ? *reinterpret_cast<const uint4*>(a.src + pos[k].off) : make_uint4(0, 0, 0, 0);
        }
#pragma unroll
        for (int k = 0; k < UPT; ++k) {
            const uint32_t d = threadIdx.x + (uint32_t)k * blockDim.x;
            if (ub + d >= a.total_units) continue;
            const uint4 out = pos[k].live ? normalize_unit(in[k], pos[k].c, a.n, a.inv[pos[k].mat]) : make_uint4(0, 0, 0, 0);
            *reinterpret_cast<uint4*>(a.dst + pos[k].off) = out;
        }
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
    if (a.dev_scalars) {            // lr and wd from device memory; d formed as the host forms it
        const float lr = a.dev_scalars[1], wd = a.dev_scalars[2];
        a.lr = lr;
        a.d = 1.0 - (double)lr * (double)wd;
    }

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

        // Flat streaming for parameters stored as they are (see the momentum kernel).
        const bool flat = !e.trans && vec && (a.np & 3) == 0;
        if (flat) {
            const int64_t nel = e.rows * e.cols;
            const int64_t e0 = tile * (T * T) + tid * 4;
            float4 wv[4];
            uint2 ov[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t idx = e0 + k * 1024;
                if (idx < nel) {
                    wv[k] = *reinterpret_cast<const float4*>(e.w + idx);
                    const int64_t xi = (a.np == e.cols) ? idx : (idx / e.cols) * a.np + idx % e.cols;
                    ov[k] = *reinterpret_cast<const uint2*>(O + xi);
                }
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t idx = e0 + k * 1024;
                if (idx >= nel) continue;
                float4 w = wv[k];
                w.x = apply_elem(w.x, bf16_to_f32(ov[k].x & 0xffffu), a.d, u);
                w.y = apply_elem(w.y, bf16_to_f32(ov[k].x >> 16), a.d, u);
                w.z = apply_elem(w.z, bf16_to_f32(ov[k].y & 0xffffu), a.d, u);
                w.w = apply_elem(w.w, bf16_to_f32(ov[k].y >> 16), a.d, u);
                *reinterpret_cast<float4*>(e.w + idx) = w;
            }
            continue;
        }
        // Interior tile: all loads first (see the momentum kernel).
        const bool full = vec && r0 + T <= e.rows && c0 + T <= e.cols && (a.np & 3) == 0;
        if (full) {
            float4 wv[4];
            uint2 ov[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = r0 + rg + 16 * i;
                wv[i] = *reinterpret_cast<const float4*>(e.w + r * e.cols + c);
                if (!e.trans) ov[i] = *reinterpret_cast<const uint2*>(O + r * a.np + c);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int64_t r = r0 + rg + 16 * i;
                float o[4];
                if (e.trans) {
#pragma unroll
                    for (int j = 0; j < 4; ++j) o[j] = bf16_to_f32(tr[cg * 4 + j][rg + 16 * i]);
                } else {
                    o[0] = bf16_to_f32(ov[i].x & 0xffffu); o[1] = bf16_to_f32(ov[i].x >> 16);
                    o[2] = bf16_to_f32(ov[i].y & 0xffffu); o[3] = bf16_to_f32(ov[i].y >> 16);
                }
                float4 w = wv[i];
                w.x = apply_elem(w.x, o[0], a.d, u);
                w.y = apply_elem(w.y, o[1], a.d, u);
                w.z = apply_elem(w.z, o[2], a.d, u);
                w.w = apply_elem(w.w, o[3], a.d, u);
                *reinterpret_cast<float4*>(e.w + r * e.cols + c) = w;
            }
        }

#pragma unroll
        for (int i = 0; i < 4 && !full; ++i) {
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

// ---------------------------------------------------------------------------------------
// Side-stream variants of the momentum, normalise and apply kernels.  While one chunk's
// Newton–Schulz products hold the compute units, the next chunk's momentum and
// normalisation and the previous chunk's apply run beside them on a second stream.  A
// product workgroup (8 waves of at most 232 VGPRs, 2 per SIMD, and about 128.5 KB of LDS)
// leaves 48 VGPRs per SIMD lane and 31.5 KB of LDS free on its CU: these kernels stay
// within that (one 16-byte unit per lane per pass, no arrays of loads in flight) and are
// launched with one workgroup per CU, so that every CU holds one product workgroup and one
// of these at once instead of the two waiting for each other.
//
// Their results are bitwise those of the kernels above: the same per-element arithmetic,
// the same tile-to-element mapping, and the momentum's sums of squares accumulated per
// tile in the same order (unit by unit, element by element, then the fixed block order).
// ---------------------------------------------------------------------------------------
// A wave-uniform double moved to scalar registers (VALU float64 instructions take it from
// there, which keeps two VGPR pairs free in the side kernels).
__device__ __forceinline__ double uniform_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// A wave-uniform 64-bit integer moved to scalar registers: the 64-bit division that finds a
// tile's matrix is expanded into vector instructions, and the table row and buffer
// resources built from its result must stay scalar.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)(uint64_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
    return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A table row with every field in scalar registers.  The row is read with vector loads (the
// compiler cannot tell that the kernel's stores leave the table alone, so the scalar cache
// is not used); buffer resources built from vector-register values would be executed in
// per-lane loops.
__device__ __forceinline__ MatEntry uniform_entry(const MatEntry* tbl, int64_t mat) {
    const MatEntry v = tbl[mat];
    MatEntry e{};
    e.w = reinterpret_cast<float*>(uniform_i64(reinterpret_cast<int64_t>(v.w)));
    e.m = reinterpret_cast<float*>(uniform_i64(reinterpret_cast<int64_t>(v.m)));
    e.g = reinterpret_cast<const void*>(uniform_i64(reinterpret_cast<int64_t>(v.g)));
    e.rows = uniform_i64(v.rows);
    e.cols = uniform_i64(v.cols);
    e.trans = (int32_t)__builtin_amdgcn_readfirstlane((uint32_t)v.trans);
    e.scale = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(v.scale)));
    return e;
}

// Four momentum elements and their NS inputs, one element after another: the scheduling
// barriers keep the four float64 chains from being interleaved, which would take more
// registers than the side kernels have.
__device__ __forceinline__ void momentum4_serial(float4& mn, uint16_t xb[4], float4 mv, const float gv[4], bool nest,
                                                 double beta, double omb) {
    mn.x = momentum_elem(mv.x, gv[0], beta, omb);
    xb[0] = x0_bits(mn.x, gv[0], nest, beta, omb);
    __builtin_amdgcn_sched_barrier(0);
    mn.y = momentum_elem(mv.y, gv[1], beta, omb);
    xb[1] = x0_bits(mn.y, gv[1], nest, beta, omb);
    __builtin_amdgcn_sched_barrier(0);
    mn.z = momentum_elem(mv.z, gv[2], beta, omb);
    xb[2] = x0_bits(mn.z, gv[2], nest, beta, omb);
    __builtin_amdgcn_sched_barrier(0);
    mn.w = momentum_elem(mv.w, gv[3], beta, omb);
    xb[3] = x0_bits(mn.w, gv[3], nest, beta, omb);
}

// Buffer accesses for the side kernels: a scalar resource per array and a 32-bit byte
// offset per lane (a generic pointer would need a 64-bit address per lane).  A chunk goes
// to these kernels only when its matrices have fewer than 2^30 elements, so every byte
// offset below fits 32 bits.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Every side-kernel access is marked non-temporal (the instructions' nt bit): the data is
// touched once per step, and streaming it through the caches with normal priority evicts
// the operand slices that the product workgroups beside it reuse.  Measured on gfx950:
// the products lose about 0.4 ms less per ladder24 step (the step 1.0 % faster, the MoE
// bucket 1.7 %).
constexpr int SIDE_CPOL = 2;
typedef float f32x4v __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 nt_ld_u2(const void* p) {
    const u32x2 v = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 nt_ld_u4(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ float4 nt_ld_f4(const float* p) {
    const f32x4v v = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(p));
    return make_float4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ void nt_st_f4(float* p, float4 f) {
    const f32x4v v = {f.x, f.y, f.z, f.w};
    __builtin_nontemporal_store(v, reinterpret_cast<f32x4v*>(p));
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t side_rsrc(const void* base, uint64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)(uint32_t)bytes, 0x00020000);
}
__device__ __forceinline__ float4 ld_f4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, SIDE_CPOL);
    return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}
__device__ __forceinline__ void st_f4(__amdgpu_buffer_rsrc_t r, uint32_t off, float4 f) {
    u32x4 v;
    v.x = __float_as_uint(f.x); v.y = __float_as_uint(f.y); v.z = __float_as_uint(f.z); v.w = __float_as_uint(f.w);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, SIDE_CPOL);
}

// Four gradient elements starting at element i, widened to float32.
template <int GDT>
__device__ __forceinline__ void side_grad4(__amdgpu_buffer_rsrc_t rg, uint32_t i, float out[4]) {
    if (GDT == MUON_DTYPE_F32) {
        const float4 v = ld_f4(rg, i * 4u);
        out[0] = v.x; out[1] = v.y; out[2] = v.z; out[3] = v.w;
    } else {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(rg, i * 2u, 0, SIDE_CPOL);
        out[0] = bf16_to_f32(v.x & 0xffffu); out[1] = bf16_to_f32(v.x >> 16);
        out[2] = bf16_to_f32(v.y & 0xffffu); out[3] = bf16_to_f32(v.y >> 16);
    }
}
template <int GDT>
__device__ __forceinline__ float side_grad1(__amdgpu_buffer_rsrc_t rg, uint32_t i) {
    if (GDT == MUON_DTYPE_F32) return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rg, i * 4u, 0, SIDE_CPOL));
    return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(rg, i * 2u, 0, SIDE_CPOL));
}

template <int GDT>
__global__ __launch_bounds__(256) void momentum_side_kernel(MomentumArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t tr[T][LDT];
    __shared__ double red[4];
    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;
    float beta32 = a.beta, omb32 = a.omb;
    if (a.dev_scalars) {
        beta32 = a.dev_scalars[0];
        omb32 = 1.0f - beta32;
    }
    const double beta = uniform_f64((double)beta32), omb = uniform_f64((double)omb32);
    const bool nest = a.nesterov != 0;
    const uint32_t np = (uint32_t)a.np;

    for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int64_t mat = uniform_i64(t / a.ew_tiles);
        const uint32_t tile = (uint32_t)(t - mat * a.ew_tiles);
        const MatEntry e = uniform_entry(a.tbl, mat);
        const uint32_t rows = (uint32_t)e.rows, cols = (uint32_t)e.cols;
        const uint32_t nel = rows * cols;
        const bool vec = (cols & 3) == 0;
        const __amdgpu_buffer_rsrc_t rm = side_rsrc(e.m, (uint64_t)nel * 4);
        const __amdgpu_buffer_rsrc_t rgr = side_rsrc(e.g, (uint64_t)nel * (GDT == MUON_DTYPE_F32 ? 4 : 2));
        const __amdgpu_buffer_rsrc_t rx = side_rsrc(a.xq + mat * a.mat_stride, (uint64_t)a.mat_stride * 2);
        double ss = 0.0;
        if (!e.trans && vec && (np & 3) == 0) {
            // flat, as in momentum_kernel
            const uint32_t e0 = tile * (T * T) + (uint32_t)tid * 4u;
#pragma unroll 1
            for (int k = 0; k < 4; ++k) {
                const uint32_t idx = e0 + (uint32_t)k * 1024u;
                if (idx >= nel) break;
                const float4 mv = ld_f4(rm, idx * 4u);
                float gv[4];
                side_grad4<GDT>(rgr, idx, gv);
                float4 mn;
                uint16_t xb[4];
                momentum4_serial(mn, xb, mv, gv, nest, beta, omb);
                st_f4(rm, idx * 4u, mn);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const double x = (double)bf16_to_f32(xb[j]);
                    ss += x * x;
                }
                const uint32_t xi = (np == cols) ? idx : (idx / cols) * np + idx % cols;
                u32x2 v;
                v.x = (uint32_t)xb[0] | ((uint32_t)xb[1] << 16);
                v.y = (uint32_t)xb[2] | ((uint32_t)xb[3] << 16);
                __builtin_amdgcn_raw_buffer_store_b64(v, rx, xi * 2u, 0, SIDE_CPOL);
            }
        } else {
            // 2-D tile, as momentum_kernel's general loop
            const uint32_t tiles_c = (cols + T - 1) / T;
            const uint32_t r0 = (tile / tiles_c) * T, c0 = (tile % tiles_c) * T;
            const uint32_t c = c0 + (uint32_t)cg * 4u;
            const int nvalid = c >= cols ? 0 : (cols - c < 4 ? (int)(cols - c) : 4);
            const bool v4 = vec && nvalid == 4;
#pragma unroll 1
            for (int i = 0; i < 4; ++i) {
                const uint32_t r = r0 + (uint32_t)rg + 16u * (uint32_t)i;
                uint16_t xb[4] = {0, 0, 0, 0};
                const bool live = r < rows && nvalid > 0;
                if (live) {
                    const uint32_t base = r * cols + c;
                    if (v4) {
                        const float4 mv = ld_f4(rm, base * 4u);
                        float gv[4];
                        side_grad4<GDT>(rgr, base, gv);
                        float4 mn;
                        momentum4_serial(mn, xb, mv, gv, nest, beta, omb);
                        st_f4(rm, base * 4u, mn);
                    } else {
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            if (j < nvalid) {
                                const uint32_t q = (base + (uint32_t)j) * 4u;
                                const float gj = side_grad1<GDT>(rgr, base + (uint32_t)j);
                                const float m0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rm, q, 0, SIDE_CPOL));
                                const float mn = momentum_elem(m0, gj, beta, omb);
                                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(mn), rm, q, 0, SIDE_CPOL);
                                xb[j] = x0_bits(mn, gj, nest, beta, omb);
                            }
                        }
                    }
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const double x = (double)bf16_to_f32(xb[j]);
                        ss += x * x;
                    }
                }
                if (!e.trans) {
                    if (live) {
                        const uint32_t xo = (r * np + c) * 2u;
                        if (nvalid == 4 && (np & 3) == 0) {
                            u32x2 v;
                            v.x = (uint32_t)xb[0] | ((uint32_t)xb[1] << 16);
                            v.y = (uint32_t)xb[2] | ((uint32_t)xb[3] << 16);
                            __builtin_amdgcn_raw_buffer_store_b64(v, rx, xo, 0, SIDE_CPOL);
                        } else {
#pragma unroll
                            for (int j = 0; j < 4; ++j)
                                if (j < nvalid) __builtin_amdgcn_raw_buffer_store_b16(xb[j], rx, xo + 2u * (uint32_t)j, 0, SIDE_CPOL);
                        }
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) tr[cg * 4 + j][rg + 16 * i] = xb[j];
                }
            }
            if (e.trans) {
                // X0 = M^T: row q of the block is column c0 + q of M
                __syncthreads();
                const int q = tid >> 2, seg = (tid & 3) * 16;
                const uint32_t xr = c0 + (uint32_t)q;
                const uint32_t xc = r0 + (uint32_t)seg;
                if (xr < cols && xc < rows) {
                    const uint32_t xo = (xr * np + xc) * 2u;
                    if (xc + 16 <= rows) {
                        const u32x4* srcv = reinterpret_cast<const u32x4*>(&tr[q][seg]);
                        __builtin_amdgcn_raw_buffer_store_b128(srcv[0], rx, xo, 0, SIDE_CPOL);
                        __builtin_amdgcn_raw_buffer_store_b128(srcv[1], rx, xo + 16u, 0, SIDE_CPOL);
                    } else {
                        for (uint32_t k = 0; xc + k < rows; ++k)
                            __builtin_amdgcn_raw_buffer_store_b16(tr[q][seg + k], rx, xo + 2u * k, 0, SIDE_CPOL);
                    }
                }
            }
        }
        ss = dev::wave_sum(ss);
        if ((tid & 63) == 0) red[tid >> 6] = ss;
        __syncthreads();
        if (tid == 0) a.partials[t] = (red[0] + red[1]) + (red[2] + red[3]);
        __syncthreads();
    }
}

// One 8-element unit per thread and pass (normalize_kernel takes UPT at a time).
__global__ __launch_bounds__(256) void normalize_side_kernel(NormalizeArgs a) {
    const uint32_t upr = (uint32_t)(a.np >> 3);
    const int64_t span = (int64_t)gridDim.x * blockDim.x;
    for (int64_t ub = (int64_t)blockIdx.x * blockDim.x; ub < a.total_units; ub += span) {
        const int64_t r0 = ub / upr;
        const uint32_t k0 = (uint32_t)(ub - r0 * upr);
        if (ub + threadIdx.x >= a.total_units) continue;
        const UnitPos pos = unit_pos(a, r0, k0, threadIdx.x, upr);
        u32x4 v = {0u, 0u, 0u, 0u};
        if (pos.live) {
            const u32x4 in = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a.src + pos.off));
            const uint4 o = normalize_unit(make_uint4(in.x, in.y, in.z, in.w), pos.c, a.n, a.inv[pos.mat]);
            v = u32x4{o.x, o.y, o.z, o.w};
        }
        __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(a.dst + pos.off));
    }
}

// Four apply elements one after another (see momentum4_serial).
__device__ __forceinline__ void apply4_serial(float4& w, const float o[4], double d, double u) {
    w.x = apply_elem(w.x, o[0], d, u);
    __builtin_amdgcn_sched_barrier(0);
    w.y = apply_elem(w.y, o[1], d, u);
    __builtin_amdgcn_sched_barrier(0);
    w.z = apply_elem(w.z, o[2], d, u);
    __builtin_amdgcn_sched_barrier(0);
    w.w = apply_elem(w.w, o[3], d, u);
}

__global__ __launch_bounds__(256) void apply_side_kernel(ApplyArgs a) {
    __shared__ __attribute__((aligned(16))) uint16_t tr[T][LDT];
    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;
    if (a.dev_scalars) {
        const float lr = a.dev_scalars[1], wd = a.dev_scalars[2];
        a.lr = lr;
        a.d = 1.0 - (double)lr * (double)wd;
    }
    const double d = uniform_f64(a.d);

    for (int64_t t = blockIdx.x; t < a.total_tiles; t += gridDim.x) {
        const int64_t mat = uniform_i64(t / a.ew_tiles);
        const int64_t tile = t - mat * a.ew_tiles;
        const MatEntry e = uniform_entry(a.tbl, mat);
        const bool vec = (e.cols & 3) == 0;
        const uint16_t* O = a.xo + mat * a.mat_stride;
        const double u = uniform_f64((double)a.lr * (double)e.scale);
        if (!e.trans && vec && (a.np & 3) == 0) {
            const uint32_t nel = (uint32_t)(e.rows * e.cols), cols = (uint32_t)e.cols;
            const uint32_t np = (uint32_t)a.np;
            const uint32_t e0 = (uint32_t)tile * (T * T) + (uint32_t)tid * 4u;
#pragma unroll 1
            for (int k = 0; k < 4; ++k) {
                const uint32_t idx = e0 + (uint32_t)k * 1024u;
                if (idx >= nel) break;
                const uint32_t xi = (np == cols) ? idx : (idx / cols) * np + idx % cols;
                const uint2 ov = nt_ld_u2(O + xi);
                float4 w = nt_ld_f4(e.w + idx);
                const float o[4] = {bf16_to_f32(ov.x & 0xffffu), bf16_to_f32(ov.x >> 16),
                                    bf16_to_f32(ov.y & 0xffffu), bf16_to_f32(ov.y >> 16)};
                apply4_serial(w, o, d, u);
                nt_st_f4(e.w + idx, w);
            }
            continue;
        }
        const int64_t tiles_c = (e.cols + T - 1) / T;
        const int64_t r0 = (tile / tiles_c) * T, c0 = (tile % tiles_c) * T;
        const int64_t c = c0 + cg * 4;
        if (e.trans) {
            const int q = tid >> 2, seg = (tid & 3) * 16;
            const int64_t orow = c0 + q;
            const int64_t ocol = r0 + seg;
            if (orow < e.cols && ocol < e.rows) {
                const uint16_t* src = O + orow * a.np + ocol;
                if (ocol + 16 <= e.rows) {
                    uint4* d4 = reinterpret_cast<uint4*>(&tr[q][seg]);
                    d4[0] = nt_ld_u4(src);
                    d4[1] = nt_ld_u4(src + 8);
                } else {
                    for (int k = 0; ocol + k < e.rows; ++k) tr[q][seg + k] = src[k];
                }
            }
            __syncthreads();
        }
#pragma unroll 1
        for (int i = 0; i < 4; ++i) {
            const int64_t r = r0 + rg + 16 * i;
            if (r >= e.rows || c >= e.cols) continue;
            const int64_t base = r * e.cols + c;
            const int nvalid = (int)((e.cols - c) < 4 ? (e.cols - c) : 4);
            float o[4] = {0.f, 0.f, 0.f, 0.f};
            if (e.trans) {
                for (int j = 0; j < nvalid; ++j) o[j] = bf16_to_f32(tr[cg * 4 + j][rg + 16 * i]);
            } else if (nvalid == 4 && (a.np & 3) == 0) {
                const uint2 v = nt_ld_u2(O + r * a.np + c);
                o[0] = bf16_to_f32(v.x & 0xffffu); o[1] = bf16_to_f32(v.x >> 16);
                o[2] = bf16_to_f32(v.y & 0xffffu); o[3] = bf16_to_f32(v.y >> 16);
            } else {
                for (int j = 0; j < nvalid; ++j) o[j] = bf16_to_f32(O[r * a.np + c + j]);
            }
            if (vec && nvalid == 4) {
                float4 w = nt_ld_f4(e.w + base);
                apply4_serial(w, o, d, u);
                nt_st_f4(e.w + base, w);
            } else {
                for (int j = 0; j < nvalid; ++j) e.w[base + j] = apply_elem(e.w[base + j], o[j], d, u);
            }
        }
        if (e.trans) __syncthreads();
    }
}

// ---------------------------------------------------------------------------------------
// AdamW for the parameters that take it.  Each operation is one float64 rounding, in the
// order below (contraction is off in this file); m and v are stored as float32.
// ---------------------------------------------------------------------------------------
struct AdamHyper {
    double lr, d, beta1, omb1, beta2, omb2, eps, bc1, bc2;
};

__device__ __forceinline__ void adam_elem(float& w, float& m, float& v, float g32, const AdamHyper& h) {
    const double g = (double)g32;
    m = (float)(h.beta1 * (double)m + h.omb1 * g);          // both products exact
    v = (float)(h.beta2 * (double)v + h.omb2 * (g * g));    // g*g exact, omb2*g^2 rounded
    const double mhat = (double)m / h.bc1;
    const double vhat = (double)v / h.bc2;
    const double den = sqrt(vhat) + h.eps;
    const double upd = (h.lr * mhat) / den;
    w = (float)(h.d * (double)w - upd);
}

__global__ __launch_bounds__(256) void adamw_kernel(AdamArgs a) {
    AdamHyper h;
    h.lr = a.lr;
    double wd = a.wd;
    h.bc1 = a.bc1;
    h.bc2 = a.bc2;
    if (a.dev_scalars) {
        h.lr = (double)a.dev_scalars[0];
        wd = (double)a.dev_scalars[1];
        h.bc1 = (double)a.dev_scalars[2];
        h.bc2 = (double)a.dev_scalars[3];
    }
    h.d = 1.0 - h.lr * wd;
    h.beta1 = a.beta1; h.omb1 = a.omb1; h.beta2 = a.beta2; h.omb2 = a.omb2; h.eps = a.eps;
    const int tid = threadIdx.x;
    for (int64_t sg = blockIdx.x; sg < a.n_segs; sg += gridDim.x) {
        const AdamSeg seg = a.segs[sg];
        const AdamEntry e = a.entries[seg.entry];
        // 4096 elements: lane l of a wave handles 16 bytes at 1 KB steps
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t idx = seg.start + k * 1024 + tid * 4;
            if (idx >= e.numel) continue;
            if (idx + 4 <= e.numel) {
                float4 w = *reinterpret_cast<const float4*>(e.w + idx);
                float4 m = *reinterpret_cast<const float4*>(e.m + idx);
                float4 v = *reinterpret_cast<const float4*>(e.v + idx);
                float g[4];
                if (e.grad_dtype == MUON_DTYPE_F32) {
                    const float4 g4 = *reinterpret_cast<const float4*>(static_cast<const float*>(e.g) + idx);
                    g[0] = g4.x; g[1] = g4.y; g[2] = g4.z; g[3] = g4.w;
                } else {
                    const uint2 g2 = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(e.g) + idx);
                    g[0] = bf16_to_f32(g2.x & 0xffffu); g[1] = bf16_to_f32(g2.x >> 16);
                    g[2] = bf16_to_f32(g2.y & 0xffffu); g[3] = bf16_to_f32(g2.y >> 16);
                }
                adam_elem(w.x, m.x, v.x, g[0], h);
                adam_elem(w.y, m.y, v.y, g[1], h);
                adam_elem(w.z, m.z, v.z, g[2], h);
                adam_elem(w.w, m.w, v.w, g[3], h);
                *reinterpret_cast<float4*>(e.w + idx) = w;
                *reinterpret_cast<float4*>(e.m + idx) = m;
                *reinterpret_cast<float4*>(e.v + idx) = v;
            } else {
                for (int64_t j = idx; j < e.numel; ++j) {
                    const float g = e.grad_dtype == MUON_DTYPE_F32 ? static_cast<const float*>(e.g)[j]
                                                                   : bf16_to_f32(static_cast<const uint16_t*>(e.g)[j]);
                    adam_elem(e.w[j], e.m[j], e.v[j], g, h);
                }
            }
        }
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

// The normalisation of several small chunks in one launch (PrepGroupArgs): the
// scale as finalize_kernel computes it, X = bf16(X0 * scale) per 16-byte unit as
// normalize_kernel computes it (padding zeroed), each matrix's units split over its
// job's `blocks` workgroups.
__global__ __launch_bounds__(256) void prep_grouped_kernel(PrepGroupArgs g) {
    __shared__ double red[5];
    const int64_t blk = blockIdx.x;
    int j = 0;
    while (j + 1 < g.n_jobs && blk >= g.job[j + 1].first) ++j;
    const PrepJob& J = g.job[j];
    const int64_t local = blk - J.first;
    const int64_t mat = local / J.blocks, part = local - mat * J.blocks;
    const double inv = block_inv(J.partials + mat * J.ew_tiles, J.ew_tiles, g.eps, red);
    const int64_t upr = J.np / 8, units = J.mp * upr;
    const int64_t per = (units + J.blocks - 1) / J.blocks;
    const int64_t u0 = part * per, u1 = units < u0 + per ? units : u0 + per;
    const int64_t base = mat * J.mp * J.np;
    for (int64_t u = u0 + threadIdx.x; u < u1; u += 256) {
        const int64_t r = u / upr, c = (u - r * upr) * 8;
        const int64_t off = base + r * J.np + c;
        uint4 o = make_uint4(0, 0, 0, 0);
        if (r < J.m && c < J.n) o = normalize_unit(*reinterpret_cast<const uint4*>(J.src + off), c, J.n, inv);
        *reinterpret_cast<uint4*>(J.dst + off) = o;
    }
}

hipError_t launch_prep_grouped(const PrepGroupArgs& g, hipStream_t s) {
    if (g.n_jobs < 1 || g.n_jobs > PREP_MAX_JOBS || g.total_blocks < 1 || g.total_blocks >= (int64_t(1) << 31))
        return hipErrorInvalidValue;
    hipLaunchKernelGGL(prep_grouped_kernel, dim3((unsigned)g.total_blocks), dim3(256), 0, s, g);
    return hipGetLastError();
}

__global__ __launch_bounds__(256) void zero_kernel(uint4* dst, uint64_t units) {
    for (uint64_t u = (uint64_t)blockIdx.x * 256 + threadIdx.x; u < units; u += (uint64_t)gridDim.x * 256)
        dst[u] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_zero(void* dst, uint64_t units, hipStream_t s) {
    if (units == 0) return hipSuccess;
    const uint64_t blocks = std::min<uint64_t>((units + 255) / 256, 2048);
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, static_cast<uint4*>(dst), units);
    return hipGetLastError();
}

hipError_t launch_finalize(const FinalizeArgs& a, int64_t count, hipStream_t s) {
    hipLaunchKernelGGL(finalize_kernel, dim3((unsigned)count), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_normalize(const NormalizeArgs& a, hipStream_t s) {
    const unsigned grid = grid_for((a.total_units + 256 * UPT - 1) / (256 * UPT), 256 * 16);
    hipLaunchKernelGGL(normalize_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_adamw(const AdamArgs& a, hipStream_t s) {
    if (a.n_segs <= 0) return hipSuccess;
    const unsigned grid = grid_for(a.n_segs);
    hipLaunchKernelGGL(adamw_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_apply(const ApplyArgs& a, hipStream_t s) {
    const unsigned grid = grid_for(a.total_tiles);
    hipLaunchKernelGGL(apply_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

// One workgroup per CU for the side-stream kernels (see above).
constexpr int64_t SIDE_GRID = 256;

hipError_t launch_momentum_side(const MomentumArgs& a, int32_t grad_dtype, hipStream_t s) {
    const unsigned grid = grid_for(a.total_tiles, SIDE_GRID);
    if (grad_dtype == MUON_DTYPE_F32)
        hipLaunchKernelGGL(momentum_side_kernel<MUON_DTYPE_F32>, dim3(grid), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL(momentum_side_kernel<MUON_DTYPE_BF16>, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_normalize_side(const NormalizeArgs& a, hipStream_t s) {
    const unsigned grid = grid_for((a.total_units + 255) / 256, SIDE_GRID);
    hipLaunchKernelGGL(normalize_side_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_apply_side(const ApplyArgs& a, hipStream_t s) {
    const unsigned grid = grid_for(a.total_tiles, SIDE_GRID);
    hipLaunchKernelGGL(apply_side_kernel, dim3(grid), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace muon
