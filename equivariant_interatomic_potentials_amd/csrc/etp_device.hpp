// etp_device.hpp -- device-side building blocks shared by the kernels:
// compile-time loops, real spherical harmonics with forward-mode
// derivatives, DPP wave reductions, XCD-aware block remapping, and
// feature-type loads (fp32 / bf16).
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>
#include <utility>

#include "etp_tables.hpp"

namespace etp {

// ------------------------------------------------------- compile-time loops
template <int I>
using ic = std::integral_constant<int, I>;

template <int B, int E, typename F>
__host__ __device__ __forceinline__ void static_range(F &&f)
{
    if constexpr (B < E) {
        [&]<int... I>(std::integer_sequence<int, I...>) __attribute__((always_inline)) {
            (f(ic<B + I>{}), ...);
        }(std::make_integer_sequence<int, E - B>{});
    }
}

// ------------------------------------------------------------- SH numbers
// Value + gradient with respect to the three components of r.
struct D3 {
    float v, g0, g1, g2;
};
__device__ __forceinline__ D3 operator+(D3 a, D3 b) { return {a.v + b.v, a.g0 + b.g0, a.g1 + b.g1, a.g2 + b.g2}; }
__device__ __forceinline__ D3 operator-(D3 a, D3 b) { return {a.v - b.v, a.g0 - b.g0, a.g1 - b.g1, a.g2 - b.g2}; }
__device__ __forceinline__ D3 operator*(float s, D3 a) { return {s * a.v, s * a.g0, s * a.g1, s * a.g2}; }
__device__ __forceinline__ D3 operator*(D3 a, D3 b)
{
    return {a.v * b.v, a.v * b.g0 + a.g0 * b.v, a.v * b.g1 + a.g1 * b.v, a.v * b.g2 + a.g2 * b.v};
}
__device__ __forceinline__ D3 d3_const(float c) { return {c, 0.f, 0.f, 0.f}; }

// Value, gradient (b), derivative along a fixed direction rho (c), and the
// gradient of that directional derivative (d): second-order forward mode for
// the Hessian-vector products of the VJP-of-VJP.
struct Jet {
    float a, b0, b1, b2, c, d0, d1, d2;
};
__device__ __forceinline__ Jet operator+(Jet x, Jet y)
{
    return {x.a + y.a, x.b0 + y.b0, x.b1 + y.b1, x.b2 + y.b2, x.c + y.c, x.d0 + y.d0, x.d1 + y.d1, x.d2 + y.d2};
}
__device__ __forceinline__ Jet operator-(Jet x, Jet y)
{
    return {x.a - y.a, x.b0 - y.b0, x.b1 - y.b1, x.b2 - y.b2, x.c - y.c, x.d0 - y.d0, x.d1 - y.d1, x.d2 - y.d2};
}
__device__ __forceinline__ Jet operator*(float s, Jet x)
{
    return {s * x.a, s * x.b0, s * x.b1, s * x.b2, s * x.c, s * x.d0, s * x.d1, s * x.d2};
}
__device__ __forceinline__ Jet operator*(Jet x, Jet y)
{
    return {x.a * y.a,
            x.a * y.b0 + x.b0 * y.a,
            x.a * y.b1 + x.b1 * y.a,
            x.a * y.b2 + x.b2 * y.a,
            x.a * y.c + x.c * y.a,
            x.a * y.d0 + x.b0 * y.c + x.c * y.b0 + x.d0 * y.a,
            x.a * y.d1 + x.b1 * y.c + x.c * y.b1 + x.d1 * y.a,
            x.a * y.d2 + x.b2 * y.c + x.c * y.b2 + x.d2 * y.a};
}
__device__ __forceinline__ Jet jet_const(float c) { return {c, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f}; }

__device__ __forceinline__ float num_const(float c, float) { return c; }
__device__ __forceinline__ D3 num_const(float c, D3) { return d3_const(c); }
__device__ __forceinline__ Jet num_const(float c, Jet) { return jet_const(c); }

// rsqrt with its derivatives applied through the number type
__device__ __forceinline__ float num_rsqrt(float s) { return rsqrtf(s); }
__device__ __forceinline__ D3 num_rsqrt(D3 s)
{
    float f = rsqrtf(s.v);
    float f1 = -0.5f * f * f * f;
    return {f, f1 * s.g0, f1 * s.g1, f1 * s.g2};
}
__device__ __forceinline__ Jet num_rsqrt(Jet s)
{
    float f = rsqrtf(s.a);
    float f3 = f * f * f;
    float f1 = -0.5f * f3;
    float f2 = 0.75f * f3 * f * f;
    return {f, f1 * s.b0, f1 * s.b1, f1 * s.b2, f1 * s.c,
            f1 * s.d0 + f2 * s.b0 * s.c, f1 * s.d1 + f2 * s.b1 * s.c, f1 * s.d2 + f2 * s.b2 * s.c};
}

constexpr double dfact_odd(int m)  // (2m-1)!!
{
    double r = 1.0;
    for (int k = 2 * m - 1; k > 1; k -= 2)
        r *= k;
    return r;
}

// Real SH in component normalisation at the unit vector (x, y, z):
//   Y_l^m = sqrt((2l+1)(l-|m|)!/(l+|m|)!) Q_l^|m|(z) * {sqrt2 Re(x+iy)^m, 1, sqrt2 Im(x+iy)^|m|}
// with Q_l^m the associated Legendre function stripped of (1-z^2)^(m/2) and
// of the Condon-Shortley phase (Q_m^m = (2m-1)!!, Q_{m+1}^m = (2m+1) z Q_m^m,
// (l-m) Q_l^m = (2l-1) z Q_{l-1}^m - (l+m-1) Q_{l-2}^m).
// The components are produced one column m at a time, emit(b, value) with
// b = l*l + l + m (a std::integral_constant), so only one column of Q and one
// power of (x + iy) are live.
template <int L, typename N, typename F>
__device__ __forceinline__ void sh_unit_emit(const N &x, const N &y, const N &z, F &&emit)
{
    N cm = num_const(1.f, x), sm = num_const(0.f, x);  // Re, Im (x + iy)^m
    static_range<0, L + 1>([&](auto m) {
        if constexpr (m > 0) {
            const N c2 = cm * x - sm * y;
            sm = sm * x + cm * y;
            cm = c2;
        }
        N q2 = num_const(0.f, x), q1 = num_const(0.f, x);  // Q_{l-2}^m, Q_{l-1}^m
        static_range<m, L + 1>([&](auto l) {
            N q;
            if constexpr (l == m) {
                q = num_const(static_cast<float>(dfact_odd(m)), x);
            } else if constexpr (l == m + 1) {
                q = static_cast<float>(2 * m + 1) * (z * q1);
            } else {
                constexpr float a = static_cast<float>((2.0 * l - 1.0) / (l - m));
                constexpr float b = static_cast<float>((l + m - 1.0) / (l - m));
                q = a * (z * q1) - b * q2;
            }
            constexpr double k0 = cx_sqrt((2.0 * l + 1.0) * cx_fact(l - m) / cx_fact(l + m));
            if constexpr (m == 0) {
                emit(std::integral_constant<int, l * l + l>{}, static_cast<float>(k0) * q);
            } else {
                constexpr float k = static_cast<float>(k0 * 1.41421356237309504880);
                emit(std::integral_constant<int, l * l + l + m>{}, k * (q * cm));
                emit(std::integral_constant<int, l * l + l - m>{}, k * (q * sm));
            }
            q2 = q1;
            q1 = q;
        });
    });
}

template <int L, typename N>
__device__ __forceinline__ void sh_unit(const N &x, const N &y, const N &z, N *Y)
{
    sh_unit_emit<L>(x, y, z, [&](auto b, const N &v) { Y[b] = v; });
}

// Y at the bond vector r (any length > 0). A zero vector gives Y = (1, 0, ...).
template <int L>
__device__ __forceinline__ void sh_value(float rx, float ry, float rz, float *Y)
{
    float r2 = rx * rx + ry * ry + rz * rz;
    float inv = r2 > 0.f ? num_rsqrt(r2) : 0.f;
    sh_unit<L>(rx * inv, ry * inv, rz * inv, Y);
    if (r2 == 0.f) {
        static_range<1, (L + 1) * (L + 1)>([&](auto b) { Y[b] = 0.f; });
        Y[0] = 1.f;
    }
}

// Y and dY/dr (gradient with respect to the unnormalised r), emitted per
// component as D3 numbers.
template <int L, typename F>
__device__ __forceinline__ void sh_grad_emit(float rx, float ry, float rz, F &&emit)
{
    D3 X{rx, 1.f, 0.f, 0.f}, Yv{ry, 0.f, 1.f, 0.f}, Z{rz, 0.f, 0.f, 1.f};
    D3 r2 = X * X + Yv * Yv + Z * Z;
    if (r2.v > 0.f) {
        D3 inv = num_rsqrt(r2);
        sh_unit_emit<L>(X * inv, Yv * inv, Z * inv, emit);
    } else {
        static_range<0, (L + 1) * (L + 1)>([&](auto b) { emit(b, d3_const(b == 0 ? 1.f : 0.f)); });
    }
}
template <int L>
__device__ __forceinline__ void sh_grad(float rx, float ry, float rz, D3 *Y)
{
    sh_grad_emit<L>(rx, ry, rz, [&](auto b, const D3 &v) { Y[b] = v; });
}

// Y, grad Y, Ydot = grad Y . rho and H rho = grad(grad Y . rho), emitted per
// component as Jet numbers.
template <int L, typename F>
__device__ __forceinline__ void sh_jet_emit(float rx, float ry, float rz, float px, float py, float pz, F &&emit)
{
    Jet X{rx, 1.f, 0.f, 0.f, px, 0.f, 0.f, 0.f};
    Jet Yv{ry, 0.f, 1.f, 0.f, py, 0.f, 0.f, 0.f};
    Jet Z{rz, 0.f, 0.f, 1.f, pz, 0.f, 0.f, 0.f};
    Jet r2 = X * X + Yv * Yv + Z * Z;
    if (r2.a > 0.f) {
        Jet inv = num_rsqrt(r2);
        sh_unit_emit<L>(X * inv, Yv * inv, Z * inv, emit);
    } else {
        static_range<0, (L + 1) * (L + 1)>([&](auto b) { emit(b, jet_const(b == 0 ? 1.f : 0.f)); });
    }
}
template <int L>
__device__ __forceinline__ void sh_jet(float rx, float ry, float rz, float px, float py, float pz, Jet *Y)
{
    sh_jet_emit<L>(rx, ry, rz, px, py, pz, [&](auto b, const Jet &v) { Y[b] = v; });
}

// ------------------------------------------------------ wave-level helpers
template <int CTRL, int ROW_MASK = 0xF, int BANK_MASK = 0xF, bool BOUND = true>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, BANK_MASK, BOUND));
}

// Sum of v over the 64 lanes; the total is exact in lane 63 (fixed order).
__device__ __forceinline__ float wave_sum_to_lane63(float v)
{
    v += dpp_mov<0xB1>(v);           // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);           // quad_perm [2,3,0,1]
    v += dpp_mov<0x141>(v);          // row_half_mirror
    v += dpp_mov<0x140>(v);          // row_mirror: every lane holds its row's sum
    v += dpp_mov<0x142, 0xA>(v);     // row_bcast:15 into rows 1 and 3
    v += dpp_mov<0x143, 0xC>(v);     // row_bcast:31 into rows 2 and 3
    return v;
}

// Wave index within the workgroup, as a wave-uniform (scalar) value.
__device__ __forceinline__ int wave_id()
{
    return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
}

__device__ __forceinline__ void wave_sync_lds()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Ends the wait for the load that produced v here: an empty asm that reads
// and writes v. A value loaded before a loop and read inside it otherwise
// keeps a loop-carried wait whose count also drains the loop's prefetches.
__device__ __forceinline__ void settle(float &v) { asm volatile("" : "+v"(v)); }

// Blocks are dispatched to the 8 XCDs round robin; this bijection gives each
// XCD a contiguous range of logical block indices (so neighbouring nodes of
// a spatially sorted graph share an L2).
__device__ __forceinline__ int xcd_remap(int b, int nb)
{
    const int q = nb >> 3, r = nb & 7, xcd = b & 7, idx = b >> 3;
    return xcd < r ? xcd * (q + 1) + idx : r * (q + 1) + (xcd - r) * q + idx;
}

// ------------------------------------------------------------ feature loads
struct bf16raw {
    uint16_t bits;
};

typedef float f32x2 __attribute__((ext_vector_type(2)));

// The CPL channels a lane owns, as one value: float for one channel, a
// two-wide vector for two (element-wise arithmetic; no packed math is
// requested from the compiler).
template <int CPL>
struct chv;
template <>
struct chv<1> {
    using type = float;
};
template <>
struct chv<2> {
    using type = f32x2;
};
template <int CPL>
using chv_t = typename chv<CPL>::type;

template <typename A, typename V>
__device__ __forceinline__ V vfma(A a, V b, V c)
{
    return a * b + c;  // contracted into fma
}

// Streaming load (read once: non-temporal) of a lane's channels.
template <typename V>
__device__ __forceinline__ V load_stream(const float *__restrict__ p)
{
    return __builtin_nontemporal_load(reinterpret_cast<const V *>(p));
}
// Cached load of a lane's channels (gathered node rows, fp32 or bf16).
template <typename V>
__device__ __forceinline__ V load_cached(const float *__restrict__ p)
{
    return *reinterpret_cast<const V *>(p);
}
template <typename V>
__device__ __forceinline__ V load_cached(const bf16raw *__restrict__ p)
{
    if constexpr (sizeof(V) == 4) {
        return __uint_as_float(static_cast<uint32_t>(reinterpret_cast<const uint16_t *>(p)[0]) << 16);
    } else {
        const uint32_t t = *reinterpret_cast<const uint32_t *>(p);
        V r;
        r.x = __uint_as_float(t << 16);
        r.y = __uint_as_float(t & 0xFFFF0000u);
        return r;
    }
}
template <typename V>
__device__ __forceinline__ void store_v(float *__restrict__ p, V v)
{
    *reinterpret_cast<V *>(p) = v;
}
template <typename V>
__device__ __forceinline__ V vzero()
{
    return V(0.f);
}

// ------------------------------------------------------ buffer resources
// Raw buffer descriptors over one contiguous block (a node's or an edge's
// rows). Lanes whose channel lies beyond C use a byte offset past the end
// of the block: the hardware's range check then returns 0 for their loads
// and drops their stores, so partially filled channel chunks need no
// branches around memory operations.
using rsrc_t = __amdgpu_buffer_rsrc_t;
constexpr uint32_t kOOB = 0x80000000u;
constexpr int kNT = 2;  // cache policy: non-temporal (streamed once)

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), static_cast<short>(0),
                                             static_cast<int>(bytes), 0x00020000);
}

// One or two f32 channels at byte offset voff (+ row offset soff) of r.
template <typename V, int AUX = 0>
__device__ __forceinline__ V bload(rsrc_t r, uint32_t voff, uint32_t soff)
{
    if constexpr (sizeof(V) == 4) {
        return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, AUX));
    } else {
        return __builtin_bit_cast(V, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, AUX));
    }
}
// One or two bf16 channels, widened to f32.
template <typename V>
__device__ __forceinline__ V bload_bf16(rsrc_t r, uint32_t voff, uint32_t soff)
{
    if constexpr (sizeof(V) == 4) {
        const uint32_t h = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
        return __uint_as_float(h << 16);
    } else {
        const uint32_t t = __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
        V v;
        v.x = __uint_as_float(t << 16);
        v.y = __uint_as_float(t & 0xFFFF0000u);
        return v;
    }
}
template <typename V, typename XT>
__device__ __forceinline__ V bload_x(rsrc_t r, uint32_t voff, uint32_t soff)
{
    if constexpr (sizeof(XT) == 2)
        return bload_bf16<V>(r, voff, soff);
    else
        return bload<V>(r, voff, soff);
}
template <typename V, int AUX = 0>
__device__ __forceinline__ void bstore(V v, rsrc_t r, uint32_t voff, uint32_t soff)
{
    if constexpr (sizeof(V) == 4) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, voff, soff, AUX);
    } else {
        typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, v), r, voff, soff, AUX);
    }
}

}  // namespace etp
