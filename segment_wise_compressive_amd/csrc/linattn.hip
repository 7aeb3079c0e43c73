// linattn.hip -- MI355X (gfx950) kernels and C ABI for linear attention with
// the feature map phi(x) = elu(x) + 1.
//
// What is computed (web pages, by title and section):
//  * "Attention Kernel Mask" (allenlu2009.github.io, 2024-11-17), "Cumsum":
//    S_t = S_{t-1} + phi(k_t), Z_t = Z_{t-1} + phi(k_t) v_t^T,
//    out_t = phi(q_t)^T Z_t / (phi(q_t) . S_t + eps), positions <= t.
//  * Same page, "How to accelerate causal linear attention": mode 3 (chunk
//    sequential: an inter-chunk term from the state of all earlier tokens plus
//    an intra-chunk masked quadratic term, then the state update) runs inside
//    every workgroup; mode 4 (scan the chunk-group states first, then run the
//    groups in parallel) splits a long sequence over workgroups.
//  * Same page, mode 2 (recurrent generation): the decode step.
//  * Same page, "Non-causal Bi-Directional Attention Kernel": one global state.
//  * "Segment-Wise Attention" (Infini-attention issue): the (Z, S) state is the
//    compressive memory carried from segment to segment.
//
// Design for CDNA4 (gfx950), in brief:
//  * One workgroup owns (head, block of DV value columns, group of tokens).
//    Each of its waves owns one 16-wide column tile of V, Z and out, so the
//    fp32 state Z of that tile lives in MFMA accumulator registers for the
//    whole token loop and never goes through LDS.
//  * q, k, v are read with 16-byte loads, phi is applied in fp32 right after
//    the load, and the results are written to LDS (double buffered, one
//    barrier per chunk) in the two layouts the MFMA operands need.
//  * All products run on 16x16 MFMA tiles.  Everything is computed in the
//    transposed orientation (rows = value column or key token, columns =
//    query token), so a lane's output column is one query token and the
//    normaliser is lane-local after a 4-lane reduction.  The accumulator of
//    one product is used directly as the operand of the next one: the score
//    tile P^T feeds P V, and the state tile Z feeds phi(Q) Z, by ordering the
//    contraction index the way the accumulator holds it (lane group g holds
//    rows 4g..4g+3 of a 16-row tile).
//  * bf16 inputs: phi(q), phi(k) and v are bf16 MFMA operands with fp32
//    accumulation.  The score tile and the state, which are fp32 sums, are
//    split into bf16 hi + lo parts (x = hi + lo to ~2^-17) so that rounding
//    them to an operand type does not cost accuracy.  The normaliser uses the
//    same rounded phi values as the numerator.  fp32 inputs use fp32 MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <math.h>

#include "linattn.h"

namespace {

typedef __bf16 bf16;
typedef bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

template <bool C, class A, class B> struct pick { typedef A type; };
template <class A, class B> struct pick<false, A, B> { typedef B type; };

// ------------------------------------------------------------------ scalar helpers
template <bool F32>
__device__ __forceinline__ float phi(float x)
{
    // elu(x) + 1 (alpha = 1): x + 1 above zero, e^x at or below it.
    if (F32) return x > 0.f ? x + 1.f : expf(x);
    return x > 0.f ? x + 1.f : __expf(x);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b)
{
    bf16x2 v = {(bf16)a, (bf16)b};  // round to nearest even (v_cvt_pk_bf16_f32)
    return __builtin_bit_cast(uint32_t, v);
}

// Raw 16-byte vector of inputs -> floats.  bf16: 8 values, fp32: 4 values.
template <bool F32> struct Vec;
template <> struct Vec<false> {
    static constexpr int N = 8;
    __device__ static void to_float(u32x4 r, float *f)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) { f[2 * i] = bf_lo(r[i]); f[2 * i + 1] = bf_hi(r[i]); }
    }
};
template <> struct Vec<true> {
    static constexpr int N = 4;
    __device__ static void to_float(u32x4 r, float *f)
    {
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = __uint_as_float(r[i]);
    }
};

// ------------------------------------------------------------------ MFMA helpers
// A "K-tile fragment" is one lane's 4 contraction values of a 16-long slice of
// the contraction index: lane (r = lane % 16, g = lane / 16) holds entries
// 4g..4g+3 for its row/column r.  This is also how a 16x16 fp32 accumulator
// holds its rows, which is what lets an accumulator be reused as an operand.
//
// bf16: v_mfma_f32_16x16x32_bf16 takes 8 values per lane, so two fragments
// (two K-tiles) are concatenated; A and B are concatenated the same way, so
// every product pairs matching contraction indices.
// fp32: v_mfma_f32_16x16x4_f32 takes 1 value per lane; fragment entry i of all
// lanes forms one K=4 step, four steps per K-tile.
__device__ __forceinline__ f32x4 mma2(f32x4 c, bf16x4 a0, bf16x4 a1, bf16x4 b0, bf16x4 b1)
{
    bf16x8 a = __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
    bf16x8 b = __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 mma1(f32x4 c, f32x4 a, f32x4 b)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x)
{
    bf16x4 r = {(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
    return r;
}

__device__ __forceinline__ f32x4 to_f32x4(bf16x4 x)
{
    f32x4 r = {(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
    return r;
}

// hi + lo split of an fp32 fragment into two bf16 fragments.
__device__ __forceinline__ void split_hi_lo(f32x4 x, bf16x4 &hi, bf16x4 &lo)
{
    hi = to_bf16x4(x);
    lo = to_bf16x4(x - to_f32x4(hi));
}

__device__ __forceinline__ float reduce_lane_groups(float x)
{
    // sum over the 4 lane groups (lanes r, r+16, r+32, r+48)
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}

// Workgroup index remapping: hardware hands consecutive workgroup ids to the
// 8 XCDs round robin.  Map them so that consecutive *logical* ids (the column
// blocks and token groups of one head) share an XCD and its L2.
__device__ __forceinline__ int xcd_remap(int id, int n)
{
    if ((n & 7) != 0) return id;
    return (id & 7) * (n >> 3) + (id >> 3);
}

// ------------------------------------------------------------------ kernel arguments
struct Args {
    const void *q, *k, *v;
    int64_t sqb, sqh, sqn, skb, skh, skn, svb, svh, svn;
    float *out;
    int64_t sob, soh, son;
    int B, H, N;
    float eps;
    const float *z_in, *s_in;
    float *z_out, *s_out;
    float *part;  // group partial states [BH][P][Gs][SLOT]
    float *fin;   // reduced states [BH][P][SLOT]
    int P;        // column blocks per head
    int G;        // token groups per head (for this launch)
    int Gs;       // partial slots per (head, column block)
    int L;        // tokens per group
};

// A slot holds one (head, column block) state: Z^T as [DV][D] (value column
// major, so a lane's 4 key rows are contiguous) followed by S [D].
template <int D, int DV> struct Slot { static constexpr int Z = DV * D, SIZE = DV * D + D; };

// LDS bytes of one workgroup: two stages of
//   phi(Q) [C][D+pad], phi(K) [C][D+pad]            (16-bit or fp32, row major)
//   phi(K)^T [D][C+pad]  x (2 for bf16: hi and lo)   (token contiguous)
//   V^T [DV][C+pad]
// plus the running key sum S (fp32, two copies).
__host__ __device__ constexpr int lds_bytes(bool f32, int d, int dv, int c)
{
    return 2 * ((2 * c * (d + (f32 ? 4 : 8)) + (f32 ? 1 : 2) * d * (c + (f32 ? 4 : 8)) + dv * (c + (f32 ? 4 : 8)))
                * (f32 ? 4 : 2)) + 2 * d * 4;
}
constexpr int LDS_LIMIT = 160 * 1024;  // per workgroup on gfx950

// ------------------------------------------------------------------ tile geometry
template <bool F32, int D, int DV, int C>
struct Geo {
    typedef typename pick<F32, float, bf16>::type E;        // LDS element
    typedef typename pick<F32, f32x4, bf16x4>::type Frag;   // K-tile fragment
    static constexpr int JT = D / 16;      // key-dimension tiles
    static constexpr int TB = C / 16;      // token tiles per chunk
    static constexpr int NW = DV / 16;     // waves = value-column tiles
    static constexpr int NT = NW * WAVE;   // threads
    static constexpr int JS = JT / NW;     // key-sum tiles owned by each wave
    static constexpr int VEC = Vec<F32>::N;
    static constexpr int PAD = 16 / (int)sizeof(E);   // 16-byte row padding
    static constexpr int RQ = D + PAD;     // row stride of phi(Q), phi(K) [token][dim]
    static constexpr int RT = C + PAD;     // row stride of phi(K)^T [dim][token], V^T [col][token]
    static constexpr int NKT = F32 ? 1 : 2;               // phi(K)^T arrays: fp32, or bf16 hi + lo
    static constexpr int OQ = 0, OK = C * RQ, OKT = 2 * C * RQ, OKL = OKT + D * RT;
    static constexpr int OVT = OKT + NKT * D * RT;
    static constexpr int STAGE = OVT + DV * RT;           // elements per stage
    static constexpr int LDS_BYTES = lds_bytes(F32, D, DV, C);
    static_assert(JT % NW == 0, "key-sum tiles must split evenly over the waves");
    static_assert(2 * STAGE * (int)sizeof(E) + 2 * D * 4 == LDS_BYTES, "LDS layout");
    // 16-byte load items per chunk
    static constexpr int IQ = C * (D / VEC);            // q rows
    static constexpr int IK = (C / 2) * (D / VEC);      // k row pairs
    static constexpr int IV = (C / 2) * (DV / VEC);     // v row pairs
    static constexpr int NQ = (IQ + NT - 1) / NT;
    static constexpr int NK = (IK + NT - 1) / NT;
    static constexpr int NV = (IV + NT - 1) / NT;
};

template <bool F32, class Frag>
__device__ __forceinline__ Frag lds_frag(const void *p)
{
    return *reinterpret_cast<const Frag *>(p);
}

__device__ __forceinline__ u32x4 ld16(const void *p) { return *reinterpret_cast<const u32x4 *>(p); }

// Load the raw q (rows), k (row pairs) and v (row pairs) of one chunk into
// registers.  Tokens at or beyond `nval` are not read.
template <bool F32, int D, int DV, int C, bool WANT_Q, bool WANT_K, bool WANT_V>
struct ChunkRegs {
    typedef Geo<F32, D, DV, C> G_;
    u32x4 q[WANT_Q ? G_::NQ : 1];
    u32x4 k[WANT_K ? 2 * G_::NK : 1];
    u32x4 v[WANT_V ? 2 * G_::NV : 1];

    __device__ __forceinline__ void load(int tid, const char *qh, const char *kh, const char *vh,
                                         int64_t sqn, int64_t skn, int64_t svn, int t0, int nval, int col0)
    {
        constexpr int ES = F32 ? 4 : 2;
        const u32x4 z = {0u, 0u, 0u, 0u};
        if (WANT_Q) {
#pragma unroll
            for (int it = 0; it < G_::NQ; ++it) {
                const int idx = tid + it * G_::NT;
                const int row = idx / (D / G_::VEC), vg = idx % (D / G_::VEC);
                q[it] = (idx < G_::IQ && row < nval)
                            ? ld16(qh + ((int64_t)(t0 + row) * sqn + vg * G_::VEC) * ES) : z;
            }
        }
        if (WANT_K) {
#pragma unroll
            for (int it = 0; it < G_::NK; ++it) {
                const int idx = tid + it * G_::NT;
                const int tp = idx / (D / G_::VEC), vg = idx % (D / G_::VEC);
                const bool ok = idx < G_::IK;
                k[2 * it] = (ok && 2 * tp < nval)
                                ? ld16(kh + ((int64_t)(t0 + 2 * tp) * skn + vg * G_::VEC) * ES) : z;
                k[2 * it + 1] = (ok && 2 * tp + 1 < nval)
                                    ? ld16(kh + ((int64_t)(t0 + 2 * tp + 1) * skn + vg * G_::VEC) * ES) : z;
            }
        }
        if (WANT_V) {
#pragma unroll
            for (int it = 0; it < G_::NV; ++it) {
                const int idx = tid + it * G_::NT;
                const int tp = idx / (DV / G_::VEC), vg = idx % (DV / G_::VEC);
                const bool ok = idx < G_::IV;
                v[2 * it] = (ok && 2 * tp < nval)
                                ? ld16(vh + ((int64_t)(t0 + 2 * tp) * svn + col0 + vg * G_::VEC) * ES) : z;
                v[2 * it + 1] = (ok && 2 * tp + 1 < nval)
                                    ? ld16(vh + ((int64_t)(t0 + 2 * tp + 1) * svn + col0 + vg * G_::VEC) * ES) : z;
            }
        }
    }

    // Apply phi and write one LDS stage.  Invalid tokens become exact zeros in
    // phi(q), phi(k) and v, so they add nothing to any product.
    //  - phi(Q), phi(K) row major: one rounding to the operand type (scores).
    //  - phi(K)^T: for bf16 as hi + lo, so the state update sees phi(k) to
    //    about 16 bits; for fp32 as is.
    //  - V^T: the input values unchanged.
    __device__ __forceinline__ void fill(int tid, typename G_::E *st, int nval, bool k_rowmajor) const
    {
        typedef typename G_::E E;
        constexpr int VEC = G_::VEC;
        if (WANT_Q) {
#pragma unroll
            for (int it = 0; it < G_::NQ; ++it) {
                const int idx = tid + it * G_::NT;
                if (idx >= G_::IQ) continue;
                const int row = idx / (D / VEC), vg = idx % (D / VEC);
                float f[VEC];
                Vec<F32>::to_float(q[it], f);
                const bool ok = row < nval;
                E *dst = st + G_::OQ + row * G_::RQ + vg * VEC;
                if (F32) {
                    f32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e) o[e] = ok ? phi<F32>(f[e]) : 0.f;
                    *reinterpret_cast<f32x4 *>(dst) = o;
                } else {
                    u32x4 o;
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        o[e] = ok ? pack_bf16(phi<F32>(f[2 * e]), phi<F32>(f[2 * e + 1])) : 0u;
                    *reinterpret_cast<u32x4 *>(dst) = o;
                }
            }
        }
        if (WANT_K) {
#pragma unroll
            for (int it = 0; it < G_::NK; ++it) {
                const int idx = tid + it * G_::NT;
                if (idx >= G_::IK) continue;
                const int tp = idx / (D / VEC), vg = idx % (D / VEC);
                float a[VEC], b[VEC];
                Vec<F32>::to_float(k[2 * it], a);
                Vec<F32>::to_float(k[2 * it + 1], b);
                const bool oka = 2 * tp < nval, okb = 2 * tp + 1 < nval;
#pragma unroll
                for (int e = 0; e < VEC; ++e) {
                    a[e] = oka ? phi<F32>(a[e]) : 0.f;
                    b[e] = okb ? phi<F32>(b[e]) : 0.f;
                }
                E *kt = st + G_::OKT + (vg * VEC) * G_::RT + 2 * tp;
                if (F32) {
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        f32x2 pr = {a[e], b[e]};
                        *reinterpret_cast<f32x2 *>(kt + e * G_::RT) = pr;
                    }
                    if (k_rowmajor) {
                        E *k0 = st + G_::OK + (2 * tp) * G_::RQ + vg * VEC;
                        f32x4 ra = {a[0], a[1], a[2], a[3]}, rb = {b[0], b[1], b[2], b[3]};
                        *reinterpret_cast<f32x4 *>(k0) = ra;
                        *reinterpret_cast<f32x4 *>(k0 + G_::RQ) = rb;
                    }
                } else {
                    bf16 ha[VEC], hb[VEC];
#pragma unroll
                    for (int e = 0; e < VEC; ++e) {
                        ha[e] = (bf16)a[e];
                        hb[e] = (bf16)b[e];
                        bf16x2 hi = {ha[e], hb[e]};
                        bf16x2 lo = {(bf16)(a[e] - (float)ha[e]), (bf16)(b[e] - (float)hb[e])};
                        *reinterpret_cast<bf16x2 *>(kt + e * G_::RT) = hi;
                        *reinterpret_cast<bf16x2 *>(kt + (G_::OKL - G_::OKT) + e * G_::RT) = lo;
                    }
                    if (k_rowmajor) {
                        E *k0 = st + G_::OK + (2 * tp) * G_::RQ + vg * VEC;
                        bf16x8 va = {ha[0], ha[1], ha[2], ha[3], ha[4], ha[5], ha[6], ha[7]};
                        bf16x8 vb = {hb[0], hb[1], hb[2], hb[3], hb[4], hb[5], hb[6], hb[7]};
                        *reinterpret_cast<bf16x8 *>(k0) = va;
                        *reinterpret_cast<bf16x8 *>(k0 + G_::RQ) = vb;
                    }
                }
            }
        }
        if (WANT_V) {
#pragma unroll
            for (int it = 0; it < G_::NV; ++it) {
                const int idx = tid + it * G_::NT;
                if (idx >= G_::IV) continue;
                const int tp = idx / (DV / VEC), vg = idx % (DV / VEC);
                E *vt = st + G_::OVT + (vg * VEC) * G_::RT + 2 * tp;
                // rows beyond nval were loaded as zeros already
                if (F32) {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        f32x2 pr = {__uint_as_float(v[2 * it][e]), __uint_as_float(v[2 * it + 1][e])};
                        *reinterpret_cast<f32x2 *>(vt + e * G_::RT) = pr;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const uint32_t wa = v[2 * it][e], wb = v[2 * it + 1][e];
                        // element 2e: low halves; element 2e+1: high halves
                        *reinterpret_cast<uint32_t *>(vt + (2 * e) * G_::RT) = (wa & 0xffffu) | (wb << 16);
                        *reinterpret_cast<uint32_t *>(vt + (2 * e + 1) * G_::RT) = (wa >> 16) | (wb & 0xffff0000u);
                    }
                }
            }
        }
    }
};

// Z += phi(K_c)^T V_c for the wave's column tile (all key tiles), and
// S += phi(K_c)^T 1 for the wave's own key-sum tiles (the all-ones B operand
// leaves S_j in exactly the lanes that hold row j of a state tile).
template <bool F32, int D, int DV, int C>
__device__ __forceinline__ void state_update(const typename Geo<F32, D, DV, C>::E *st, int w, int r, int g,
                                             f32x4 *Zacc, f32x4 *Sown)
{
    typedef Geo<F32, D, DV, C> G_;
    typedef typename G_::E E;
    const E *kt = st + G_::OKT;
    const E *vt = st + G_::OVT + (16 * w + r) * G_::RT + 4 * g;
    if (F32) {
        const f32x4 ones = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int sa = 0; sa < G_::TB; ++sa) {
            const f32x4 vb = lds_frag<F32, f32x4>(vt + 16 * sa);
#pragma unroll
            for (int jt = 0; jt < G_::JT; ++jt) {
                const f32x4 ka = lds_frag<F32, f32x4>(kt + (16 * jt + r) * G_::RT + 16 * sa + 4 * g);
                Zacc[jt] = mma1(Zacc[jt], ka, vb);
            }
#pragma unroll
            for (int js = 0; js < G_::JS; ++js) {
                const int jt = w * G_::JS + js;
                const f32x4 ka = lds_frag<F32, f32x4>(kt + (16 * jt + r) * G_::RT + 16 * sa + 4 * g);
                Sown[js] = mma1(Sown[js], ka, ones);
            }
        }
    } else {
        const bf16 one = (bf16)1.f, zr = (bf16)0.f;
        const bf16x4 ones = {one, one, one, one};
        const bf16x4 zero = {zr, zr, zr, zr};
        const E *kl = st + G_::OKL;
#pragma unroll
        for (int sa = 0; sa < G_::TB; sa += 2) {
            const bool two = sa + 1 < G_::TB;
            const bf16x4 vb0 = lds_frag<F32, bf16x4>(vt + 16 * sa);
            const bf16x4 vb1 = two ? lds_frag<F32, bf16x4>(vt + 16 * (sa + 1)) : zero;
#pragma unroll
            for (int jt = 0; jt < G_::JT; ++jt) {
                const int o = (16 * jt + r) * G_::RT + 16 * sa + 4 * g;
                const bf16x4 h0 = lds_frag<F32, bf16x4>(kt + o), l0 = lds_frag<F32, bf16x4>(kl + o);
                const bf16x4 h1 = two ? lds_frag<F32, bf16x4>(kt + o + 16) : zero;
                const bf16x4 l1 = two ? lds_frag<F32, bf16x4>(kl + o + 16) : zero;
                Zacc[jt] = mma2(Zacc[jt], h0, h1, vb0, vb1);
                Zacc[jt] = mma2(Zacc[jt], l0, l1, vb0, vb1);
            }
#pragma unroll
            for (int js = 0; js < G_::JS; ++js) {
                const int o = (16 * (w * G_::JS + js) + r) * G_::RT + 16 * sa + 4 * g;
                const bf16x4 h0 = lds_frag<F32, bf16x4>(kt + o), l0 = lds_frag<F32, bf16x4>(kl + o);
                const bf16x4 h1 = two ? lds_frag<F32, bf16x4>(kt + o + 16) : zero;
                const bf16x4 l1 = two ? lds_frag<F32, bf16x4>(kl + o + 16) : zero;
                Sown[js] = mma2(Sown[js], h0, h1, ones, ones);
                Sown[js] = mma2(Sown[js], l0, l1, ones, ones);
            }
        }
    }
}

// ------------------------------------------------------------------ kernels
// Partial state of one token group: Z_g = phi(K_g)^T V_g (the wave's column
// tile), S_g = sum phi(k) (the wave's key-sum tiles).  Written to the group's
// slot.
template <bool F32, int D, int DV, int C>
__global__ void __launch_bounds__(DV / 16 * WAVE) k_group_state(const Args a)
{
    typedef Geo<F32, D, DV, C> G_;
    typedef typename G_::E E;
    __shared__ __attribute__((aligned(16))) char smem_raw[G_::LDS_BYTES];
    E *smem = reinterpret_cast<E *>(smem_raw);
    const int tid = threadIdx.x, w = tid / WAVE, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int p = wg % a.P, rest = wg / a.P, grp = rest % a.G, bh = rest / a.G;
    const int b = bh / a.H, h = bh % a.H;
    const int t_begin = grp * a.L, t_end = min(t_begin + a.L, a.N);
    constexpr int ES = F32 ? 4 : 2;
    const char *kh = (const char *)a.k + (b * a.skb + h * a.skh) * ES;
    const char *vh = (const char *)a.v + (b * a.svb + h * a.svh) * ES;

    f32x4 Zacc[G_::JT], Sown[G_::JS];
#pragma unroll
    for (int jt = 0; jt < G_::JT; ++jt) Zacc[jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int js = 0; js < G_::JS; ++js) Sown[js] = (f32x4){0.f, 0.f, 0.f, 0.f};

    ChunkRegs<F32, D, DV, C, false, true, true> R;
    const int nch = (t_end - t_begin + C - 1) / C;
    R.load(tid, nullptr, kh, vh, 0, a.skn, a.svn, t_begin, min(C, t_end - t_begin), p * DV);
    R.fill(tid, smem, min(C, t_end - t_begin), false);
    for (int ch = 0; ch < nch; ++ch) {
        __syncthreads();
        const int t0 = t_begin + ch * C;
        const bool more = ch + 1 < nch;
        const int nnext = more ? min(C, t_end - t0 - C) : 0;
        if (more) R.load(tid, nullptr, kh, vh, 0, a.skn, a.svn, t0 + C, nnext, p * DV);
        const E *st = smem + (ch & 1) * G_::STAGE;
        state_update<F32, D, DV, C>(st, w, r, g, Zacc, Sown);
        if (more) R.fill(tid, smem + ((ch + 1) & 1) * G_::STAGE, nnext, false);
    }

    constexpr int SL = Slot<D, DV>::SIZE;
    float *slot = a.part + ((int64_t)(bh * a.P + p) * a.Gs + grp) * SL;
#pragma unroll
    for (int jt = 0; jt < G_::JT; ++jt)
        *reinterpret_cast<f32x4 *>(slot + (16 * w + r) * D + 16 * jt + 4 * g) = Zacc[jt];
    if (r == 0) {
#pragma unroll
        for (int js = 0; js < G_::JS; ++js)
            *reinterpret_cast<f32x4 *>(slot + Slot<D, DV>::Z + 16 * (w * G_::JS + js) + 4 * g) = Sown[js];
    }
}

// Sum of the group partials in group order (plus the carried-in state):
//  * to_state = true : state-only causal call -> z_out, s_out ([j][c] layout).
//  * to_state = false: non-causal call -> reduced slots `fin`.
// Every element is read and written by the same thread, so z_out may be z_in.
template <int D, int DV>
__global__ void __launch_bounds__(256) k_reduce(const Args a, int ngroups, bool to_state)
{
    constexpr int SL = Slot<D, DV>::SIZE, SZ = Slot<D, DV>::Z;
    const int bh = blockIdx.x;
    const int total = a.P * SL;
    for (int e = threadIdx.x; e < total; e += blockDim.x) {
        const int p = e / SL, kk = e % SL;
        const bool is_s = kk >= SZ;
        if (to_state && is_s && p != 0) continue;  // S is identical in every column block
        int64_t sidx;
        float acc;
        if (!is_s) {
            const int c = kk / D, j = kk % D;
            sidx = (int64_t)bh * D * D + (int64_t)j * D + p * DV + c;
            acc = (to_state && a.z_in) ? a.z_in[sidx] : 0.f;
        } else {
            sidx = (int64_t)bh * D + (kk - SZ);
            acc = (to_state && a.s_in) ? a.s_in[sidx] : 0.f;
        }
        const float *src = a.part + (int64_t)(bh * a.P + p) * a.Gs * SL + kk;
        for (int gi = 0; gi < ngroups; ++gi) acc += src[(int64_t)gi * SL];
        if (to_state) {
            if (!is_s) { if (a.z_out) a.z_out[sidx] = acc; }
            else if (a.s_out) a.s_out[sidx] = acc;
        } else {
            a.fin[(int64_t)(bh * a.P + p) * SL + kk] = acc;
        }
    }
}

// Chunk-sequential forward of one token group (mode 3 inside the group).
// CAUSAL: out_t = [phi(q_t) Z_prev + sum_{s<=t in chunk} P_ts v_s] /
//                 [phi(q_t) . S_prev + sum_{s<=t in chunk} P_ts + eps],
//         P = phi(Q_c) phi(K_c)^T, then Z += phi(K_c)^T V_c, S += phi(K_c)^T 1.
//         The group starts from z_in/s_in plus the partials of all earlier
//         groups (mode 4); the last group writes z_out/s_out.
// !CAUSAL (non-causal apply): out_t = phi(q_t) Z / (phi(q_t) . S + eps) with
//         the reduced global state.
template <bool F32, int D, int DV, int C, bool CAUSAL>
__global__ void __launch_bounds__(DV / 16 * WAVE) k_chunk_fwd(const Args a)
{
    typedef Geo<F32, D, DV, C> G_;
    typedef typename G_::E E;
    typedef typename G_::Frag Frag;
    constexpr int JT = G_::JT, TB = G_::TB, JS = G_::JS;
    constexpr int ES = F32 ? 4 : 2;
    constexpr int SL = Slot<D, DV>::SIZE;
    __shared__ __attribute__((aligned(16))) char smem_raw[G_::LDS_BYTES];
    E *smem = reinterpret_cast<E *>(smem_raw);
    float *sS = reinterpret_cast<float *>(smem_raw + 2 * G_::STAGE * sizeof(E));  // [2][D]

    const int tid = threadIdx.x, w = tid / WAVE, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int p = wg % a.P, rest = wg / a.P, grp = rest % a.G, bh = rest / a.G;
    const int b = bh / a.H, h = bh % a.H;
    const int t_begin = grp * a.L, t_end = min(t_begin + a.L, a.N);
    const int col = p * DV + 16 * w + r;  // this lane's value column (state layout)
    const char *qh = (const char *)a.q + (b * a.sqb + h * a.sqh) * ES;
    const char *kh = (const char *)a.k + (b * a.skb + h * a.skh) * ES;
    const char *vh = (const char *)a.v + (b * a.svb + h * a.svh) * ES;
    float *oh = a.out + b * a.sob + h * a.soh;

    // ---- starting state of this group: Z tile of this wave's columns, and
    // this wave's share of S (published to LDS for every wave)
    f32x4 Zacc[JT], Sown[JS];
    if (CAUSAL) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 16 * jt + 4 * g + i;
                Zacc[jt][i] = a.z_in ? a.z_in[(int64_t)bh * D * D + (int64_t)j * D + col] : 0.f;
            }
        }
#pragma unroll
        for (int js = 0; js < JS; ++js) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int j = 16 * (w * JS + js) + 4 * g + i;
                Sown[js][i] = a.s_in ? a.s_in[(int64_t)bh * D + j] : 0.f;
            }
        }
        const float *slots = a.part + (int64_t)(bh * a.P + p) * a.Gs * SL;
        for (int gp = 0; gp < grp; ++gp) {
            const float *sl = slots + (int64_t)gp * SL;
#pragma unroll
            for (int jt = 0; jt < JT; ++jt)
                Zacc[jt] += *reinterpret_cast<const f32x4 *>(sl + (16 * w + r) * D + 16 * jt + 4 * g);
#pragma unroll
            for (int js = 0; js < JS; ++js)
                Sown[js] += *reinterpret_cast<const f32x4 *>(sl + Slot<D, DV>::Z + 16 * (w * JS + js) + 4 * g);
        }
    } else {
        const float *sl = a.fin + (int64_t)(bh * a.P + p) * SL;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
            Zacc[jt] = *reinterpret_cast<const f32x4 *>(sl + (16 * w + r) * D + 16 * jt + 4 * g);
#pragma unroll
        for (int js = 0; js < JS; ++js)
            Sown[js] = *reinterpret_cast<const f32x4 *>(sl + Slot<D, DV>::Z + 16 * (w * JS + js) + 4 * g);
    }
    if (r == 0) {
#pragma unroll
        for (int js = 0; js < JS; ++js)
            *reinterpret_cast<f32x4 *>(sS + 16 * (w * JS + js) + 4 * g) = Sown[js];
    }

    ChunkRegs<F32, D, DV, C, true, CAUSAL, CAUSAL> R;
    const int nch = (t_end - t_begin + C - 1) / C;
    R.load(tid, qh, kh, vh, a.sqn, a.skn, a.svn, t_begin, min(C, t_end - t_begin), p * DV);
    R.fill(tid, smem, min(C, t_end - t_begin), true);

    for (int ch = 0; ch < nch; ++ch) {
        __syncthreads();
        const int t0 = t_begin + ch * C;
        const int nval = min(C, t_end - t0);
        const bool more = ch + 1 < nch;
        const int nnext = more ? min(C, t_end - t0 - C) : 0;
        if (more) R.load(tid, qh, kh, vh, a.sqn, a.skn, a.svn, t0 + C, nnext, p * DV);
        const E *st = smem + (ch & 1) * G_::STAGE;

        // running key sum before this chunk, for the lane's key rows
        f32x4 Sv[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
            Sv[jt] = *reinterpret_cast<const f32x4 *>(sS + (ch & 1) * D + 16 * jt + 4 * g);

        // state as the A operand of phi(Q) Z: hi (+ lo for bf16)
        Frag zh[JT], zl[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            if (F32) {
                zh[jt] = *reinterpret_cast<const Frag *>(&Zacc[jt]);
            } else {
                bf16x4 hi, lo;
                split_hi_lo(Zacc[jt], hi, lo);
                zh[jt] = *reinterpret_cast<const Frag *>(&hi);
                zl[jt] = *reinterpret_cast<const Frag *>(&lo);
            }
        }

#pragma unroll
        for (int tb = 0; tb < TB; ++tb) {
            // phi(q) fragments of query token 16*tb + r, dims 16*jt + 4g..+3
            Frag qf[JT];
            float dp = 0.f;
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                qf[jt] = lds_frag<F32, Frag>(st + G_::OQ + (16 * tb + r) * G_::RQ + 16 * jt + 4 * g);
                f32x4 qv;
                if (F32) qv = *reinterpret_cast<const f32x4 *>(&qf[jt]);
                else qv = to_f32x4(*reinterpret_cast<const bf16x4 *>(&qf[jt]));
#pragma unroll
                for (int i = 0; i < 4; ++i) dp += qv[i] * Sv[jt][i];
            }
            f32x4 o = {0.f, 0.f, 0.f, 0.f};
            // inter-chunk term: O^T += Z^T phi(Q)^T
            if (F32) {
#pragma unroll
                for (int jt = 0; jt < JT; ++jt)
                    o = mma1(o, *reinterpret_cast<const f32x4 *>(&zh[jt]), *reinterpret_cast<const f32x4 *>(&qf[jt]));
            } else {
#pragma unroll
                for (int jt = 0; jt < JT; jt += 2) {
                    const bf16x4 *zh4 = reinterpret_cast<const bf16x4 *>(zh);
                    const bf16x4 *zl4 = reinterpret_cast<const bf16x4 *>(zl);
                    const bf16x4 *q4 = reinterpret_cast<const bf16x4 *>(qf);
                    o = mma2(o, zh4[jt], zh4[jt + 1], q4[jt], q4[jt + 1]);
                    o = mma2(o, zl4[jt], zl4[jt + 1], q4[jt], q4[jt + 1]);
                }
            }
            float rs = 0.f;
            if (CAUSAL) {
                // intra-chunk term over key tiles sa <= tb
                const E *vrow = st + G_::OVT + (16 * w + r) * G_::RT + 4 * g;
                if (F32) {
#pragma unroll
                    for (int sa = 0; sa <= tb; ++sa) {
                        f32x4 pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int jt = 0; jt < JT; ++jt) {
                            const f32x4 kf = lds_frag<F32, f32x4>(st + G_::OK + (16 * sa + r) * G_::RQ + 16 * jt + 4 * g);
                            pt = mma1(pt, kf, *reinterpret_cast<const f32x4 *>(&qf[jt]));
                        }
                        if (sa == tb) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) if (4 * g + i > r) pt[i] = 0.f;
                        }
                        rs += (pt[0] + pt[1]) + (pt[2] + pt[3]);
                        o = mma1(o, lds_frag<F32, f32x4>(vrow + 16 * sa), pt);
                    }
                } else {
                    const bf16x4 zero = {(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
                    const bf16x4 *q4 = reinterpret_cast<const bf16x4 *>(qf);
#pragma unroll
                    for (int sa = 0; sa <= tb; sa += 2) {
                        const bool two = sa + 1 <= tb;
                        f32x4 pt0 = {0.f, 0.f, 0.f, 0.f}, pt1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                        for (int jt = 0; jt < JT; jt += 2) {
                            const E *k0 = st + G_::OK + (16 * sa + r) * G_::RQ + 16 * jt + 4 * g;
                            pt0 = mma2(pt0, lds_frag<F32, bf16x4>(k0), lds_frag<F32, bf16x4>(k0 + 16), q4[jt], q4[jt + 1]);
                            if (two) {
                                const E *k1 = k0 + 16 * G_::RQ;
                                pt1 = mma2(pt1, lds_frag<F32, bf16x4>(k1), lds_frag<F32, bf16x4>(k1 + 16), q4[jt], q4[jt + 1]);
                            }
                        }
                        // causal mask inside the diagonal tile: key 4g+i > query r
                        if (sa == tb) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) if (4 * g + i > r) pt0[i] = 0.f;
                        }
                        if (two && sa + 1 == tb) {
#pragma unroll
                            for (int i = 0; i < 4; ++i) if (4 * g + i > r) pt1[i] = 0.f;
                        }
                        rs += (pt0[0] + pt0[1]) + (pt0[2] + pt0[3]);
                        if (two) rs += (pt1[0] + pt1[1]) + (pt1[2] + pt1[3]);
                        bf16x4 ph0, pl0, ph1 = zero, pl1 = zero;
                        split_hi_lo(pt0, ph0, pl0);
                        if (two) split_hi_lo(pt1, ph1, pl1);
                        const bf16x4 va0 = lds_frag<F32, bf16x4>(vrow + 16 * sa);
                        const bf16x4 va1 = two ? lds_frag<F32, bf16x4>(vrow + 16 * (sa + 1)) : zero;
                        o = mma2(o, va0, va1, ph0, ph1);
                        o = mma2(o, va0, va1, pl0, pl1);
                    }
                }
            }
            const float den = reduce_lane_groups(dp + rs) + a.eps;
            const int tq = 16 * tb + r;
            if (tq < nval) {
                const float inv = 1.f / den;
                f32x4 res = o * inv;
                *reinterpret_cast<f32x4 *>(oh + (int64_t)(t0 + tq) * a.son + p * DV + 16 * w + 4 * g) = res;
            }
        }

        if (CAUSAL) {
            state_update<F32, D, DV, C>(st, w, r, g, Zacc, Sown);
            if (r == 0) {
#pragma unroll
                for (int js = 0; js < JS; ++js)
                    *reinterpret_cast<f32x4 *>(sS + ((ch + 1) & 1) * D + 16 * (w * JS + js) + 4 * g) = Sown[js];
            }
        } else if (r == 0) {
#pragma unroll
            for (int js = 0; js < JS; ++js)
                *reinterpret_cast<f32x4 *>(sS + ((ch + 1) & 1) * D + 16 * (w * JS + js) + 4 * g) = Sown[js];
        }
        if (more) R.fill(tid, smem + ((ch + 1) & 1) * G_::STAGE, nnext, true);
    }

    if (CAUSAL && grp == a.G - 1) {
        if (a.z_out) {
#pragma unroll
            for (int jt = 0; jt < JT; ++jt)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a.z_out[(int64_t)bh * D * D + (int64_t)(16 * jt + 4 * g + i) * D + col] = Zacc[jt][i];
        }
        if (a.s_out && p == 0 && r == 0) {
#pragma unroll
            for (int js = 0; js < JS; ++js)
                *reinterpret_cast<f32x4 *>(a.s_out + (int64_t)bh * D + 16 * (w * JS + js) + 4 * g) = Sown[js];
        }
    }
}

// One recurrent step for every head: Z += phi(k) v^T, S += phi(k),
// out = phi(q)^T Z / (phi(q) . S + eps).  Pure streaming over Z (read, update,
// write back once); every state element is read and written by one thread.
template <bool F32, int D>
__global__ void __launch_bounds__(256) k_decode(const void *qp, const void *kp, const void *vp,
                                                float *z, float *s, float *out, int BH, float eps)
{
    constexpr int QD = D / 4;            // column quads
    constexpr int RPT = 16;              // rows per thread
    constexpr int RG = D / RPT;          // row groups
    constexpr int TPH = QD * RG;         // threads per head
    constexpr int HPB = 256 / TPH;       // heads per block
    __shared__ float sphik[HPB][D], sphiq[HPB][D];
    __shared__ f32x4 red[HPB][RG][QD];
    __shared__ float dred[HPB][RG];

    const int tid = threadIdx.x, hl = tid / TPH, lt = tid % TPH;
    const int bh = blockIdx.x * HPB + hl;
    const bool active = bh < BH;
    const int cq = lt % QD, rg = lt / QD;

    auto ld = [&](const void *base, int64_t i) -> float {
        if (F32) return ((const float *)base)[i];
        const uint16_t u = ((const uint16_t *)base)[i];
        return __uint_as_float((uint32_t)u << 16);
    };
    if (active) {
        for (int j = lt; j < D; j += TPH) {
            sphik[hl][j] = phi<F32>(ld(kp, (int64_t)bh * D + j));
            sphiq[hl][j] = phi<F32>(ld(qp, (int64_t)bh * D + j));
        }
    }
    __syncthreads();
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float dpart = 0.f;
    if (active) {
        f32x4 vv;
#pragma unroll
        for (int e = 0; e < 4; ++e) vv[e] = ld(vp, (int64_t)bh * D + 4 * cq + e);
        float *zh = z + (int64_t)bh * D * D + 4 * cq;
        f32x4 zr[RPT];
#pragma unroll
        for (int m = 0; m < RPT; ++m) zr[m] = *reinterpret_cast<const f32x4 *>(zh + (int64_t)(m * RG + rg) * D);
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int j = m * RG + rg;
            const float fj = sphik[hl][j];
            zr[m] += fj * vv;
            *reinterpret_cast<f32x4 *>(zh + (int64_t)j * D) = zr[m];
            acc += sphiq[hl][j] * zr[m];
        }
        if (cq == 0) {
#pragma unroll
            for (int m = 0; m < RPT; ++m) {
                const int j = m * RG + rg;
                const float sj = s[(int64_t)bh * D + j] + sphik[hl][j];
                s[(int64_t)bh * D + j] = sj;
                dpart += sphiq[hl][j] * sj;
            }
        }
    }
    red[hl][rg][cq] = acc;
    if (cq == 0) dred[hl][rg] = dpart;
    __syncthreads();
    if (active && rg == 0) {
        f32x4 tot = red[hl][0][cq];
        float den = dred[hl][0];
#pragma unroll
        for (int i = 1; i < RG; ++i) { tot += red[hl][i][cq]; den += dred[hl][i]; }
        den += eps;
        *reinterpret_cast<f32x4 *>(out + (int64_t)bh * D + 4 * cq) = tot * (1.f / den);
    }
}

// ------------------------------------------------------------------ host side
inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

bool overlaps(const void *a, size_t na, const void *b, size_t nb)
{
    if (!a || !b || na == 0 || nb == 0) return false;
    const char *pa = (const char *)a, *pb = (const char *)b;
    return pa < pb + nb && pb < pa + na;
}

// Columns per workgroup: one 16-wide tile per wave, at most 4 waves.
inline int cols_per_wg(int d) { return d < 64 ? d : 64; }

template <bool F32, int D, int DV, int C>
constexpr bool fits() { return lds_bytes(F32, D, DV, C) <= LDS_LIMIT; }

// Largest supported chunk <= requested whose LDS fits one workgroup.
int pick_chunk(bool f32, int d, int chunk)
{
    if (chunk == 0) chunk = f32 ? 32 : 64;
    const int cands[4] = {128, 64, 32, 16};
    for (int c : cands)
        if (c <= chunk && lds_bytes(f32, d, cols_per_wg(d), c) <= LDS_LIMIT) return c;
    return 16;
}

struct Plan {
    int C, DV, P, G, L, Gs;
    size_t slot_floats;
    size_t part_off, part_bytes, fin_off, fin_bytes, copy_off, copy_bytes, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Token groups: enough workgroups to cover the chip (about one per CU), each
// group a whole number of chunks, at most 32 groups per head.
int pick_groups(int64_t units, int N, int C, int target)
{
    if (N <= 0) return 1;
    int64_t maxg = (N + C - 1) / C;
    int64_t g = (target + units - 1) / units;
    if (g < 1) g = 1;
    if (g > maxg) g = maxg;
    if (g > 32) g = 32;
    return (int)g;
}

Plan plan_causal(int B, int H, int N, int d, la_dtype dt, int chunk, int flags, bool want_out)
{
    Plan pl;
    const bool f32 = dt == LA_F32;
    pl.C = pick_chunk(f32, d, chunk);
    pl.DV = cols_per_wg(d);
    pl.P = d / pl.DV;
    const int64_t BH = (int64_t)B * H;
    pl.G = pick_groups(BH * pl.P, N, pl.C, want_out ? 256 : 512);
    int64_t per = (N + pl.G - 1) / pl.G;
    pl.L = (int)(((per + pl.C - 1) / pl.C) * pl.C);
    if (pl.L < pl.C) pl.L = pl.C;
    pl.G = N > 0 ? (int)((N + pl.L - 1) / pl.L) : 1;
    pl.Gs = want_out ? pl.G - 1 : pl.G;
    pl.slot_floats = (size_t)pl.DV * d + d;
    pl.part_off = 0;
    pl.part_bytes = align256((size_t)BH * pl.P * pl.Gs * pl.slot_floats * 4);
    pl.fin_off = pl.part_off + pl.part_bytes;
    pl.fin_bytes = 0;
    pl.copy_off = pl.fin_off;
    pl.copy_bytes = (want_out && (flags & LA_WS_INPLACE_STATE)) ? align256((size_t)BH * ((size_t)d * d + d) * 4) : 0;
    pl.total = pl.copy_off + pl.copy_bytes;
    if (N == 0) pl.total = pl.copy_bytes, pl.part_bytes = 0, pl.copy_off = 0, pl.Gs = 0;
    return pl;
}

Plan plan_noncausal(int B, int H, int N, int d, la_dtype dt)
{
    Plan pl;
    const bool f32 = dt == LA_F32;
    pl.C = pick_chunk(f32, d, 0);
    pl.DV = cols_per_wg(d);
    pl.P = d / pl.DV;
    const int64_t BH = (int64_t)B * H;
    pl.G = pick_groups(BH * pl.P, N, pl.C, 512);
    int64_t per = (N + pl.G - 1) / pl.G;
    pl.L = (int)(((per + pl.C - 1) / pl.C) * pl.C);
    if (pl.L < pl.C) pl.L = pl.C;
    pl.G = N > 0 ? (int)((N + pl.L - 1) / pl.L) : 1;
    pl.Gs = pl.G;
    pl.slot_floats = (size_t)pl.DV * d + d;
    pl.part_off = 0;
    pl.part_bytes = align256((size_t)BH * pl.P * pl.Gs * pl.slot_floats * 4);
    pl.fin_off = pl.part_bytes;
    pl.fin_bytes = align256((size_t)BH * pl.P * pl.slot_floats * 4);
    pl.copy_off = pl.fin_off + pl.fin_bytes;
    pl.copy_bytes = 0;
    pl.total = pl.copy_off;
    if (N == 0) pl.total = 0;
    return pl;
}

// ---- kernel dispatch tables (dtype x d x chunk)
typedef void (*KFn)(Args);

template <bool F32, int D, int C>
void launch_group_state(const Args &a, int nwg, hipStream_t st)
{
    constexpr int DV = D < 64 ? D : 64;
    if constexpr (fits<F32, D, DV, C>())
        hipLaunchKernelGGL((k_group_state<F32, D, DV, C>), dim3(nwg), dim3(Geo<F32, D, DV, C>::NT), 0, st, a);
}

template <bool F32, int D, int C, bool CAUSAL>
void launch_chunk(const Args &a, int nwg, hipStream_t st)
{
    constexpr int DV = D < 64 ? D : 64;
    if constexpr (fits<F32, D, DV, C>())
        hipLaunchKernelGGL((k_chunk_fwd<F32, D, DV, C, CAUSAL>), dim3(nwg), dim3(Geo<F32, D, DV, C>::NT), 0, st, a);
}

template <bool F32, int D>
void dispatch_c(int C, int what, const Args &a, int nwg, hipStream_t st)
{
    // what: 0 = group state, 1 = causal chunk, 2 = non-causal apply
#define LA_CASE(CC)                                                          \
    case CC:                                                                 \
        if (what == 0) launch_group_state<F32, D, CC>(a, nwg, st);           \
        else if (what == 1) launch_chunk<F32, D, CC, true>(a, nwg, st);      \
        else launch_chunk<F32, D, CC, false>(a, nwg, st);                    \
        break;
    switch (C) {
        LA_CASE(16)
        LA_CASE(32)
        LA_CASE(64)
        LA_CASE(128)
    default: break;
    }
#undef LA_CASE
}

void dispatch(bool f32, int d, int C, int what, const Args &a, int nwg, hipStream_t st)
{
    if (f32) {
        if (d == 32) dispatch_c<true, 32>(C, what, a, nwg, st);
        else if (d == 64) dispatch_c<true, 64>(C, what, a, nwg, st);
        else dispatch_c<true, 128>(C, what, a, nwg, st);
    } else {
        if (d == 32) dispatch_c<false, 32>(C, what, a, nwg, st);
        else if (d == 64) dispatch_c<false, 64>(C, what, a, nwg, st);
        else dispatch_c<false, 128>(C, what, a, nwg, st);
    }
}

void launch_reduce(int d, const Args &a, int BH, int ngroups, bool to_state, hipStream_t st)
{
    if (d == 32) hipLaunchKernelGGL((k_reduce<32, 32>), dim3(BH), dim3(256), 0, st, a, ngroups, to_state);
    else if (d == 64) hipLaunchKernelGGL((k_reduce<64, 64>), dim3(BH), dim3(256), 0, st, a, ngroups, to_state);
    else hipLaunchKernelGGL((k_reduce<128, 64>), dim3(BH), dim3(256), 0, st, a, ngroups, to_state);
}

la_status check_common(int B, int H, int N, int d, la_dtype dt, float eps)
{
    if (B < 0 || H < 0 || N < 0) return LA_ERR_SHAPE;
    if (dt != LA_F32 && dt != LA_BF16) return LA_ERR_DTYPE;
    if (d != 32 && d != 64 && d != 128) return LA_ERR_UNSUPPORTED;
    if (!(eps >= 0.f) || !isfinite(eps)) return LA_ERR_VALUE;
    // 32-bit workgroup and token indexing
    if ((int64_t)B * H > (1 << 24) || N > (1 << 30)) return LA_ERR_SHAPE;
    return LA_OK;
}

la_status check_tensor(const void *p, la_strides s, size_t es)
{
    if (!p) return LA_ERR_NULL;
    if (!aligned16(p)) return LA_ERR_ALIGN;
    if (s.b < 0 || s.h < 0 || s.n < 0) return LA_ERR_SHAPE;
    if (((size_t)s.b * es) % 16 || ((size_t)s.h * es) % 16 || ((size_t)s.n * es) % 16) return LA_ERR_ALIGN;
    return LA_OK;
}

Args make_args(const void *q, la_strides sq, const void *k, la_strides sk, const void *v, la_strides sv,
               float *out, la_strides so, int B, int H, int N, float eps)
{
    Args a;
    memset(&a, 0, sizeof(a));
    a.q = q; a.k = k; a.v = v;
    a.sqb = sq.b; a.sqh = sq.h; a.sqn = sq.n;
    a.skb = sk.b; a.skh = sk.h; a.skn = sk.n;
    a.svb = sv.b; a.svh = sv.h; a.svn = sv.n;
    a.out = out; a.sob = so.b; a.soh = so.h; a.son = so.n;
    a.B = B; a.H = H; a.N = N; a.eps = eps;
    return a;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char *la_status_str(la_status s)
{
    switch (s) {
    case LA_OK: return "LA_OK";
    case LA_ERR_NULL: return "LA_ERR_NULL: a required pointer is NULL";
    case LA_ERR_SHAPE: return "LA_ERR_SHAPE: negative or too large size or stride";
    case LA_ERR_DTYPE: return "LA_ERR_DTYPE: dtype must be LA_F32 or LA_BF16";
    case LA_ERR_ALIGN: return "LA_ERR_ALIGN: pointers and strides must be 16-byte aligned";
    case LA_ERR_UNSUPPORTED: return "LA_ERR_UNSUPPORTED: d must be 32, 64 or 128 and chunk 0, 16, 32, 64 or 128";
    case LA_ERR_VALUE: return "LA_ERR_VALUE: eps must be finite and >= 0";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
    case LA_ERR_ALIAS: return "LA_ERR_ALIAS: output state overlaps an input state";
    case LA_ERR_LAUNCH: return "LA_ERR_LAUNCH: a HIP launch failed";
    }
    return "unknown la_status";
}

int la_version(void) { return 100; }

size_t la_causal_fwd_workspace(int B, int H, int N, int d, la_dtype dt, int chunk, int flags)
{
    if (check_common(B, H, N, d, dt, 0.f) != LA_OK) return 0;
    if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return 0;
    // the larger of the with-output and state-only plans
    Plan a = plan_causal(B, H, N, d, dt, chunk, flags, true);
    Plan b = plan_causal(B, H, N, d, dt, chunk, flags, false);
    return a.total > b.total ? a.total : b.total;
}

la_status la_causal_fwd(const void *q, la_strides sq, const void *k, la_strides sk,
                        const void *v, la_strides sv, la_dtype dt,
                        float *out, la_strides so,
                        int B, int H, int N, int d, int chunk, float eps,
                        const float *z_in, const float *s_in,
                        float *z_out, float *s_out,
                        void *workspace, size_t ws_bytes, void *hip_stream)
{
    la_status st = check_common(B, H, N, d, dt, eps);
    if (st != LA_OK) return st;
    if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return LA_ERR_UNSUPPORTED;
    const size_t es = dt == LA_F32 ? 4 : 2;
    const bool want_out = out != nullptr;
    if (!want_out && !z_out && !s_out) return LA_ERR_NULL;
    if (N > 0) {
        if ((st = check_tensor(q, sq, es)) != LA_OK) return st;
        if ((st = check_tensor(k, sk, es)) != LA_OK) return st;
        if ((st = check_tensor(v, sv, es)) != LA_OK) return st;
        if (want_out && (st = check_tensor(out, so, 4)) != LA_OK) return st;
    }
    for (const void *p : {(const void *)z_in, (const void *)s_in, (const void *)z_out, (const void *)s_out})
        if (p && !aligned16(p)) return LA_ERR_ALIGN;
    const int64_t BH = (int64_t)B * H;
    const size_t zb = (size_t)BH * d * d * 4, sb = (size_t)BH * d * 4;
    // outputs may equal inputs exactly, nothing else may overlap
    if (z_out && z_in && z_out != (float *)z_in && overlaps(z_out, zb, z_in, zb)) return LA_ERR_ALIAS;
    if (s_out && s_in && s_out != (float *)s_in && overlaps(s_out, sb, s_in, sb)) return LA_ERR_ALIAS;
    if (overlaps(z_out, zb, s_in, sb) || overlaps(s_out, sb, z_in, zb) || overlaps(z_out, zb, s_out, sb))
        return LA_ERR_ALIAS;
    const bool z_inplace = z_out && z_out == z_in, s_inplace = s_out && s_out == s_in;
    const int flags = (z_inplace || s_inplace) ? LA_WS_INPLACE_STATE : 0;
    Plan pl = plan_causal(B, H, N, d, dt, chunk, flags, want_out);
    if (ws_bytes < pl.total || (pl.total > 0 && !workspace)) return LA_ERR_WORKSPACE;
    if (BH == 0) return LA_OK;

    hipStream_t stream = (hipStream_t)hip_stream;
    (void)hipGetLastError();
    char *ws = (char *)workspace;
    Args a = make_args(q, sq, k, sk, v, sv, out, so, B, H, N, eps);
    a.z_in = z_in; a.s_in = s_in; a.z_out = z_out; a.s_out = s_out;
    a.P = pl.P; a.L = pl.L; a.Gs = pl.Gs;
    a.part = (float *)(ws + pl.part_off);
    const bool f32 = dt == LA_F32;

    if (N == 0 || !want_out) {
        // state only: group partials over all groups, then the ordered sum
        // with the carried-in state (same thread reads and writes each element)
        if (N > 0) {
            a.G = pl.G;
            dispatch(f32, d, pl.C, 0, a, (int)(BH * pl.P * pl.G), stream);
        }
        launch_reduce(d, a, (int)BH, N > 0 ? pl.G : 0, true, stream);
        return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
    }

    // in-place state with more than one reader of the input state: read it
    // from a copy in the workspace
    if ((z_inplace || s_inplace) && (pl.G > 1 || pl.P > 1)) {
        float *cz = (float *)(ws + pl.copy_off);
        float *cs = cz + (size_t)BH * d * d;
        if (z_inplace) {
            if (hipMemcpyAsync(cz, z_in, zb, hipMemcpyDeviceToDevice, stream) != hipSuccess) return LA_ERR_LAUNCH;
            a.z_in = cz;
        }
        if (s_inplace) {
            if (hipMemcpyAsync(cs, s_in, sb, hipMemcpyDeviceToDevice, stream) != hipSuccess) return LA_ERR_LAUNCH;
            a.s_in = cs;
        }
    }
    if (pl.G > 1) {
        a.G = pl.G - 1;  // partials of groups 0 .. G-2
        dispatch(f32, d, pl.C, 0, a, (int)(BH * pl.P * (pl.G - 1)), stream);
    }
    a.G = pl.G;
    dispatch(f32, d, pl.C, 1, a, (int)(BH * pl.P * pl.G), stream);
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

la_status la_decode_step(const void *q, const void *k, const void *v, la_dtype dt,
                         float *z, float *s, float *out,
                         int B, int H, int d, float eps, void *hip_stream)
{
    la_status st = check_common(B, H, 1, d, dt, eps);
    if (st != LA_OK) return st;
    if (!q || !k || !v || !z || !s || !out) return LA_ERR_NULL;
    for (const void *p : {q, k, v, (const void *)z, (const void *)s, (const void *)out})
        if (!aligned16(p)) return LA_ERR_ALIGN;
    const int64_t BH = (int64_t)B * H;
    if (BH == 0) return LA_OK;
    hipStream_t stream = (hipStream_t)hip_stream;
    (void)hipGetLastError();
    const int hpb = 256 / ((d / 4) * (d / 16));
    const int nblk = (int)((BH + hpb - 1) / hpb);
    const bool f32 = dt == LA_F32;
#define LA_DEC(F, DD) hipLaunchKernelGGL((k_decode<F, DD>), dim3(nblk), dim3(256), 0, stream, q, k, v, z, s, out, (int)BH, eps)
    if (f32) { if (d == 32) LA_DEC(true, 32); else if (d == 64) LA_DEC(true, 64); else LA_DEC(true, 128); }
    else { if (d == 32) LA_DEC(false, 32); else if (d == 64) LA_DEC(false, 64); else LA_DEC(false, 128); }
#undef LA_DEC
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

size_t la_noncausal_workspace(int B, int H, int N, int d, la_dtype dt)
{
    if (check_common(B, H, N, d, dt, 0.f) != LA_OK) return 0;
    return plan_noncausal(B, H, N, d, dt).total;
}

la_status la_noncausal_fwd(const void *q, la_strides sq, const void *k, la_strides sk,
                           const void *v, la_strides sv, la_dtype dt,
                           float *out, la_strides so,
                           int B, int H, int N, int d, float eps,
                           void *workspace, size_t ws_bytes, void *hip_stream)
{
    la_status st = check_common(B, H, N, d, dt, eps);
    if (st != LA_OK) return st;
    const size_t es = dt == LA_F32 ? 4 : 2;
    if (N > 0) {
        if ((st = check_tensor(q, sq, es)) != LA_OK) return st;
        if ((st = check_tensor(k, sk, es)) != LA_OK) return st;
        if ((st = check_tensor(v, sv, es)) != LA_OK) return st;
        if ((st = check_tensor(out, so, 4)) != LA_OK) return st;
    }
    Plan pl = plan_noncausal(B, H, N, d, dt);
    if (ws_bytes < pl.total || (pl.total > 0 && !workspace)) return LA_ERR_WORKSPACE;
    const int64_t BH = (int64_t)B * H;
    if (BH == 0 || N == 0) return LA_OK;
    hipStream_t stream = (hipStream_t)hip_stream;
    (void)hipGetLastError();
    char *ws = (char *)workspace;
    Args a = make_args(q, sq, k, sk, v, sv, out, so, B, H, N, eps);
    a.P = pl.P; a.Gs = pl.Gs;
    a.part = (float *)(ws + pl.part_off);
    a.fin = (float *)(ws + pl.fin_off);
    const bool f32 = dt == LA_F32;
    // 1) partial states of the token groups, 2) ordered reduction per head,
    // 3) every query against the global state (token groups of L_apply)
    a.G = pl.G; a.L = pl.L;
    dispatch(f32, d, pl.C, 0, a, (int)(BH * pl.P * pl.G), stream);
    launch_reduce(d, a, (int)BH, pl.G, false, stream);
    const int la = pl.C * 4;
    a.L = la;
    a.G = (N + la - 1) / la;
    dispatch(f32, d, pl.C, 2, a, (int)(BH * pl.P * a.G), stream);
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

}  // extern "C"
