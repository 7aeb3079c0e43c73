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
//  * Causal forward, one launch: a workgroup owns (head, block of DV value
//    columns, group of tokens).  It publishes its group's partial state
//    (device-visible stores, then a per-call 64-bit tag as the flag), and sums
//    the published states of the earlier groups of its head (the state before
//    the group).  Workgroups only wait for lower-indexed ones of the same XCD,
//    which the hardware dispatches first.
//  * bf16 inputs at d = 64 and 128 (k_cs_fwd): each of the 4 waves owns 16
//    value columns for the whole group, so its slice of the state never
//    leaves its registers.  q, k and v stay in registers for two passes: a
//    state-only pass publishes the group's partial state early, then the
//    outputs are computed chunk by chunk; the earlier groups' state is summed
//    after the first chunk, which is corrected, and later chunks run against
//    the full prefix.  Only psi = phi - 1 (bf16) enters the MFMAs; the
//    all-ones part of phi is carried in fp32 (see k_cs_fwd).
//  * Other dtype / d pairs (k_chunk_fwd): the 4 waves share the state through
//    LDS (Z^T as bf16 hi + lo parts, S as an extra row) and each wave owns one
//    16-row query tile; the published state is summed before the chunk loop.
//  * All products run on 16x16 MFMA tiles in the transposed orientation
//    (rows = value column or key token, columns = query token): the score
//    tile P^T feeds P V directly, and the accumulator layout (lane group g
//    holds rows 4g..4g+3) is the operand layout of the next product.  The
//    gfx950 LDS transpose read supplies token-major operands.
//  * The fp32 sums fed back as operands (scores, state) are split into bf16
//    hi + lo parts; fp32 inputs use fp32 MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <time.h>
#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <stdlib.h>

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
    // elu(x) + 1 (alpha = 1): x + 1 above zero, e^x at or below it.  Since
    // e^x >= x + 1 everywhere, this is max(x + 1, min(e^x, 1)): four
    // instructions (the min is the clamp bit of v_exp_f32), and the
    // NaN-propagating maximum keeps phi(NaN) = NaN, phi(+inf) = +inf,
    // phi(-inf) = 0.  e^x = 2^(x log2 e) to about 2 ulp.
    const float e = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x * 1.44269504088896340736f), 0.f, 1.f);
    return __builtin_elementwise_maximum(x + 1.f, e);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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
// every product pairs matching contraction indices (mma8 below).
// fp32: v_mfma_f32_16x16x4_f32 takes 1 value per lane; fragment entry i of all
// lanes forms one K=4 step, four steps per K-tile.

__device__ __forceinline__ f32x4 mma1(f32x4 c, f32x4 a, f32x4 b)
{
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[0], b[0], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[1], b[1], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[2], b[2], c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(a[3], b[3], c, 0, 0, 0);
    return c;
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
    float *part;  // per (head, column block) state slots [BH][P][NS][SLOT]
    float *fin;   // reduced states [BH][P][SLOT]
    int P;        // column blocks per head
    int G;        // token groups per head (for this launch)
    int NS;       // slots per (head, column block)
    int L;        // tokens per group
    int slot0;    // slot written by group 0 of a group-state launch
    // single-pass causal kernel: one flag per (head, column block, group),
    // set to `epoch` (unique per call) when that group's slot is published
    unsigned long long *flags;
    unsigned long long epoch;
    unsigned long long wait_tag;   // the tag waits look for (== epoch)
    int spin_limit;                // polls before a wait gives up
    unsigned *giveups;             // counter of waits that gave up (workspace offset 0)
    int wait_s;   // s_out is s_in and shared by P > 1 column blocks
    int unnorm;   // causal outputs without the normaliser (numerators only)
    int direct;   // k_cs_state with one share: write z_out = z_in + Z (no slot)
};

// A slot holds one (head, column block) state in the layout of the state
// tensors: Z[:, block columns] as [D][DV] (key row major) followed by S [D].
template <int D, int DV> struct Slot { static constexpr int Z = DV * D, SIZE = DV * D + D; };

// ------------------------------------------------------------------ tile geometry
constexpr int NWAVE = 4;                 // waves per workgroup
constexpr int NTHR = NWAVE * WAVE;       // threads per workgroup

__host__ __device__ constexpr int pad_of(bool f32) { return f32 ? 4 : 8; }  // 16 bytes of row padding

// LDS bytes of one workgroup (one chunk stage, row major as loaded):
//   phi(K) [C][D]            (x2 for bf16: hi and lo parts)
//   V      [C][DV]           (the input values)
//   Z^T    [DV+1][D+pad]     (x2 for bf16: hi and lo parts): the shared state
//                            and S as row DV
// bf16 phi(K) and V rows are unpadded with their 16-byte pieces XOR-swizzled
// (see swz_piece); fp32 rows and Z^T rows carry 16 bytes of padding.
__host__ __device__ constexpr int kv_row(bool f32, int w) { return f32 ? w + pad_of(true) : w; }
__host__ __device__ constexpr int lds_bytes(bool f32, int d, int dv, int c)
{
    return ((f32 ? 1 : 2) * c * kv_row(f32, d) + c * kv_row(f32, dv) +
            (f32 ? 1 : 2) * (dv + 1) * (d + pad_of(f32))) * (f32 ? 4 : 2);
}
constexpr int LDS_LIMIT = 160 * 1024;  // per workgroup on gfx950
// workgroups per CU the causal kernel's register budget is sized for
__host__ __device__ constexpr int minwg_of(bool /*f32*/, int d, int c) { return (d <= 64 && c == 64) ? (d == 64 ? 2 : 3) : 1; }
// Register-resident groups (64-token chunks): chunks a workgroup keeps in
// registers, and the workgroups per CU its register budget is sized for.
__host__ __device__ constexpr int res_cpg(bool f32, int d) { return d == 128 ? (f32 ? 1 : 2) : (f32 && d == 64 ? 2 : 4); }
__host__ __device__ constexpr int res_minwg(bool f32, int d) { return (d == 128 || (f32 && d == 64)) ? 1 : 2; }

template <bool F32, int D, int DV, int C>
struct Geo {
    typedef typename pick<F32, float, bf16>::type E;      // LDS element
    static constexpr int JT = D / 16;      // key-dimension tiles
    static constexpr int CT = DV / 16;     // value-column tiles
    static constexpr int TBN = C / 16;     // token tiles per chunk
    static constexpr int BPW = TBN / NWAVE;  // query tiles per wave (1 or 2)
    static constexpr int ZT = JT * CT / NWAVE;  // state tiles owned by each wave
    static constexpr int SMAX = (JT + NWAVE - 1) / NWAVE;  // key-sum tiles per wave (at most)
    static constexpr int VEC = Vec<F32>::N;  // values per 16-byte vector
    static constexpr int PAD = pad_of(F32);
    static constexpr int RK = kv_row(F32, D);   // row stride of phi(K) [token][dim]
    static constexpr int RV = kv_row(F32, DV);  // row stride of V [token][col]
    static constexpr int RZ = D + PAD;          // row stride of Z^T [col][dim]
    static constexpr int NP = F32 ? 1 : 2; // copies of phi(K) and Z^T (hi, lo)
    static constexpr int OK = 0, OKL = C * RK, OV = NP * C * RK;
    static constexpr int ZR = DV + 1;                      // rows of Z^T: state, then S
    static constexpr int OZ = OV + C * RV, OZL = OZ + ZR * RZ;
    static constexpr int NE = OZ + NP * ZR * RZ;           // E elements in all
    static constexpr int LDS_BYTES = lds_bytes(F32, D, DV, C);
    static_assert(NE * (int)sizeof(E) == LDS_BYTES, "LDS layout");
    // register pipeline depth: chunk c+DEPTH is loaded while chunk c is
    // computed.  With output stores in the same loop, the gfx9 memory counter
    // cannot separate older loads from newer ones, so a deeper register
    // pipeline would only add registers; latency is hidden by occupancy.
    static constexpr int DEPTH = 1;

    static_assert(TBN % NWAVE == 0 && (BPW == 1 || BPW == 2), "chunk must be 64 or 128 tokens");
    static_assert((JT * CT) % NWAVE == 0, "state tiles must split evenly over the waves");
    // 16-byte load items per chunk (rows x vectors)
    static constexpr int IK = C * (D / VEC);
    static constexpr int IV = C * (DV / VEC);
    static constexpr int NK = (IK + NTHR - 1) / NTHR;
    static constexpr int NV = (IV + NTHR - 1) / NTHR;
    // per-lane 16-byte vectors of one query row (dims: bf16 32u+8g..+7, fp32 16u+4g..+3)
    static constexpr int NQV = F32 ? JT : JT / 2;
};

typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

// ---- MFMA operand fragments.
// Contraction over the head dimension (scores, inter-chunk term): A and B are
// read "naturally" -- bf16: 8 consecutive dims 32u + 8g .. +7 per lane; fp32:
// 4 dims 16u + 4g .. +3.  Contraction over tokens (P V, state update): the
// operand must hold 4 consecutive tokens of one column, which is how a 16x16
// accumulator holds its rows; it is read from the row-major [token][col]
// arrays with the gfx950 LDS transpose read (bf16) or four scalar reads (fp32).

// bf16: 8 natural values at `p` (16-byte aligned).
__device__ __forceinline__ bf16x8 nat8(const bf16 *p) { return *reinterpret_cast<const bf16x8 *>(p); }
__device__ __forceinline__ f32x4 nat4(const float *p) { return *reinterpret_cast<const f32x4 *>(p); }

// bf16 [row][W] arrays of phi(K) and V: the 16-byte piece p of a row is stored
// at piece p ^ f(row).  gfx950 LDS has 64 banks (256 bytes per clock): a
// 16-byte read is served 16 lanes at a time, an 8-byte read 32 lanes at a
// time.  f spreads both ways these arrays are read over all 64 banks:
// 16-byte reads of one piece from 16 consecutive rows (scores, inter term),
// and transpose reads of two pieces from each of 8 consecutive rows.
//   256-byte rows: f = 2 (row & 7) + ((row >> 3) & 1)
//   128-byte rows: f = 2 ((row >> 1) & 3) + ((row >> 3) & 1)   (rows of one
//                  parity share a 256-byte bank cycle)
//    64-byte rows: f = 2 ((row >> 2) & 1) + ((row >> 3) & 1)   (4 rows per
//                  bank cycle)
// The transpose read of four pieces per row (state update) stays 2-way.
template <int W>
__device__ __forceinline__ int swz_piece(int row, int piece)
{
    if constexpr (W == 32) return piece ^ (2 * ((row >> 2) & 1) + ((row >> 3) & 1));
    else if constexpr (W == 64) return piece ^ (2 * ((row >> 1) & 3) + ((row >> 3) & 1));
    else if constexpr (W == 128) return piece ^ (2 * (row & 7) + ((row >> 3) & 1));
    else return piece;   // padded fp32 rows: not swizzled
}
// element offset of (row, col) in a swizzled bf16 [row][W] array (col % 4 == 0)
template <int W>
__device__ __forceinline__ int swz(int row, int col) { return row * W + swz_piece<W>(row, col >> 3) * 8 + (col & 7); }

// bf16 transposed fragment: lane (n = lane % 16, g = lane / 16) receives rows
// s0 + 4g .. s0 + 4g + 3 of column col0 + n of a swizzled [row][W] array.
// Each lane addresses row s0 + 4g + n/4, columns col0 + 4(n%4) .. +3; the
// transpose read redistributes those 4-element pieces within every 16 lanes.
template <int W>
__device__ __forceinline__ bf16x4 tr4(const bf16 *base, int s0, int col0, int n, int g)
{
    const bf16 *p = base + swz<W>(s0 + 4 * g + (n >> 2), col0 + 4 * (n & 3));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(bf16 *)p);
}
// two tiles (s0 and s0 + 16) concatenated: the 8 values of one bf16 MFMA
template <int W>
__device__ __forceinline__ bf16x8 tr8(const bf16 *base, int s0, int col0, int n, int g)
{
    const bf16x4 a = tr4<W>(base, s0, col0, n, g), b = tr4<W>(base, s0 + 16, col0, n, g);
    return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
// fp32 transposed fragment: rows s0 + 4g + i of column col0 + n.
__device__ __forceinline__ f32x4 trf(const float *base, int ld, int s0, int col0, int n, int g)
{
    f32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = base[(s0 + 4 * g + i) * ld + col0 + n];
    return v;
}

__device__ __forceinline__ f32x4 mma8(f32x4 c, bf16x8 a, bf16x8 b)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---- buffer access.  Every q/k/v/out access goes through a buffer resource
// whose base is advanced per chunk with scalar arithmetic; lanes add a fixed
// 32-bit offset.  Reads past the end of the resource return zero.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int RSRC_FLAGS = 0x00020000;   // raw (untyped) buffer, dword access

__device__ __forceinline__ rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const int n = bytes <= 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : (int)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, n, RSRC_FLAGS);
}
__device__ __forceinline__ u32x4 bload16(rsrc_t r, uint32_t off) { return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0); }
__device__ __forceinline__ void bstore16(rsrc_t r, uint32_t off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, 0);
}
// Streaming variants, with the non-temporal cache policy: for data touched
// once (q, k, v of the column-split and non-causal kernels, the causal
// outputs), so that it does not displace what stays in the caches -- the
// published states that the look-back reads from L2.  Measured: 8% faster
// causal calls, 9% faster non-causal (whose outputs are better stored
// normally).
constexpr int CPOL_STREAM = 2;   // nt
__device__ __forceinline__ u32x4 bload16nt(rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL_STREAM);
}
__device__ __forceinline__ void bstore16nt(rsrc_t r, uint32_t off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, CPOL_STREAM);
}

// A head's rows [t0, end of tensor): a view that buffer accesses index by
// (row - t0) * stride + column bytes.
struct RowView {
    const char *head;   // element (row 0, col 0) of the head
    int64_t rs;         // row stride in bytes
    int64_t span;       // bytes from `head` to the end of the head's last row
    __device__ __forceinline__ rsrc_t at(int t0) const { return make_rsrc(head + t0 * rs, span - t0 * rs); }
    // rows from t0 if `live`, else an empty resource (reads return zero
    // without touching memory, writes are dropped)
    __device__ __forceinline__ rsrc_t at(int t0, bool live) const
    {
        return make_rsrc(head + t0 * rs, live ? span - t0 * rs : 0);
    }
};
// a lane offset that is out of range for every resource (the access is dropped)
constexpr uint32_t OFF_NONE = 0xfffffff0u;

// bf16 pair <-> packed word; hi/lo split of two floats into two packed words
__device__ __forceinline__ uint32_t pk_bf16(float a, float b)
{
    bf16x2 v = {(bf16)a, (bf16)b};  // round to nearest even
    return __builtin_bit_cast(uint32_t, v);
}
// returns {hi word, lo word}: hi = a and b rounded to bf16 (nearest even:
// the scores use hi alone, so it must be unbiased), lo = the remainders
// rounded to bf16; hi + lo carries ~17 significant bits
__device__ __forceinline__ uint2 split_pk(float a, float b)
{
    const uint32_t hi = pk_bf16(a, b);
    // hi.low16 << 16 through v_perm_b32 (bytes: 0, 0, hi.b0, hi.b1), so that
    // the compiler reuses hi instead of converting a again
    const float ah = __uint_as_float(__builtin_amdgcn_perm(hi, hi, 0x05040c0cu));
    return make_uint2(hi, pk_bf16(a - ah, b - bf_hi(hi)));
}

// Query rows of one wave tile: lane (r, g) holds query token r of the tile and
// the dims it supplies as an MFMA operand, so phi(q) never goes through LDS.
template <bool F32, int D>
struct QRegs {
    static constexpr int NQV = F32 ? D / 16 : D / 32;
    u32x4 raw[NQV];

    __device__ __forceinline__ static int dim0(int u, int g) { return F32 ? 16 * u + 4 * g : 32 * u + 8 * g; }
    // byte offsets of the lane's vectors within a chunk view
    __device__ __forceinline__ static void offsets(uint32_t *off, int row, int64_t rs, int g)
    {
        constexpr int ES = F32 ? 4 : 2;
#pragma unroll
        for (int u = 0; u < NQV; ++u) off[u] = (uint32_t)(row * rs + dim0(u, g) * ES);
    }
    __device__ __forceinline__ void load(rsrc_t r, const uint32_t *off)
    {
#pragma unroll
        for (int u = 0; u < NQV; ++u) raw[u] = bload16(r, off[u]);
    }
};

// Cooperative load of the k and v rows of one chunk into registers
// (16-byte vectors, consecutive threads along a row), then phi and the LDS
// stage.  Rows at or beyond `nval` are zeroed in fill().
template <bool F32, int D, int DV, int C>
struct KVRegs {
    typedef Geo<F32, D, DV, C> G_;
    static_assert(G_::IK % NTHR == 0 && G_::IV % NTHR == 0, "whole load items per thread");
    u32x4 k[G_::NK];
    u32x4 v[G_::NV];

    __device__ __forceinline__ static void offsets(uint32_t *ko, uint32_t *vo, int tid, int64_t krs, int64_t vrs)
    {
#pragma unroll
        for (int it = 0; it < G_::NK; ++it) {
            const int idx = tid + it * NTHR;
            ko[it] = (uint32_t)((idx / (D / G_::VEC)) * krs + (idx % (D / G_::VEC)) * 16);
        }
#pragma unroll
        for (int it = 0; it < G_::NV; ++it) {
            const int idx = tid + it * NTHR;
            vo[it] = (uint32_t)((idx / (DV / G_::VEC)) * vrs + (idx % (DV / G_::VEC)) * 16);
        }
    }
    __device__ __forceinline__ void load(rsrc_t kr, rsrc_t vr, const uint32_t *ko, const uint32_t *vo)
    {
#pragma unroll
        for (int it = 0; it < G_::NK; ++it) k[it] = bload16(kr, ko[it]);
#pragma unroll
        for (int it = 0; it < G_::NV; ++it) v[it] = bload16(vr, vo[it]);
    }

    // phi(K): bf16 hi + lo (the state update sees phi(k) to ~16 bits; the
    // scores use hi), or fp32.  V: the input values unchanged.
    // Rows at or past `nval` were loaded as zeros (reads past the end of a
    // resource), which V keeps; phi(K) must be zero there (phi(0) = 1), which
    // only a ragged chunk needs.
    __device__ __forceinline__ void fill(int tid, typename G_::E *st, int nval) const
    {
        if (nval >= C) fill_rows<false>(tid, st, C);
        else fill_rows<true>(tid, st, nval);
    }

    // bf16 only: phi(K) split into hi + lo once (kh, kl), for chunks staged
    // twice (the group's own state, then the chunk loop); stage() then only
    // copies registers to LDS.
    u32x4 kh[G_::NK], kl[G_::NK];
    __device__ __forceinline__ void phi_split(int tid, int nval)
    {
#pragma unroll
        for (int it = 0; it < G_::NK; ++it) {
            const int row = (tid + it * NTHR) / (D / G_::VEC);
            const bool ok = nval >= C || row < nval;
            float f[G_::VEC];
            Vec<F32>::to_float(k[it], f);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint2 sp_ = split_pk(ok ? phi<F32>(f[2 * e]) : 0.f, ok ? phi<F32>(f[2 * e + 1]) : 0.f);
                kh[it][e] = sp_.x;
                kl[it][e] = sp_.y;
            }
        }
    }
    __device__ __forceinline__ void stage(int tid, typename G_::E *st) const
    {
        typedef typename G_::E E;
        constexpr int VEC = G_::VEC;
#pragma unroll
        for (int it = 0; it < G_::NK; ++it) {
            const int idx = tid + it * NTHR;
            const int row = idx / (D / VEC), vg = idx % (D / VEC);
            E *dst = st + G_::OK + row * G_::RK + swz_piece<G_::RK>(row, vg) * VEC;
            *reinterpret_cast<u32x4 *>(dst) = kh[it];
            *reinterpret_cast<u32x4 *>(dst + (G_::OKL - G_::OK)) = kl[it];
        }
#pragma unroll
        for (int it = 0; it < G_::NV; ++it) {
            const int idx = tid + it * NTHR;
            const int row = idx / (DV / VEC), vg = idx % (DV / VEC);
            *reinterpret_cast<u32x4 *>(st + G_::OV + row * G_::RV + swz_piece<G_::RV>(row, vg) * VEC) = v[it];
        }
    }
    template <bool MASK>
    __device__ __forceinline__ void fill_rows(int tid, typename G_::E *st, int nval) const
    {
        typedef typename G_::E E;
        constexpr int VEC = G_::VEC;
#pragma unroll
        for (int it = 0; it < G_::NK; ++it) {
            const int idx = tid + it * NTHR;
            const int row = idx / (D / VEC), vg = idx % (D / VEC);
            float f[VEC];
            Vec<F32>::to_float(k[it], f);
            const bool ok = !MASK || row < nval;
            E *dst = st + G_::OK + row * G_::RK + (F32 ? vg : swz_piece<G_::RK>(row, vg)) * VEC;
#pragma unroll
            for (int e = 0; e < VEC; ++e) f[e] = ok ? phi<F32>(f[e]) : 0.f;
            if (F32) {
                *reinterpret_cast<f32x4 *>(dst) = (f32x4){f[0], f[1], f[2], f[3]};
            } else {
                u32x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) { const uint2 sp_ = split_pk(f[2 * e], f[2 * e + 1]); hi[e] = sp_.x; lo[e] = sp_.y; }
                *reinterpret_cast<u32x4 *>(dst) = hi;
                *reinterpret_cast<u32x4 *>(dst + (G_::OKL - G_::OK)) = lo;
            }
        }
#pragma unroll
        for (int it = 0; it < G_::NV; ++it) {
            const int idx = tid + it * NTHR;
            const int row = idx / (DV / VEC), vg = idx % (DV / VEC);
            *reinterpret_cast<u32x4 *>(st + G_::OV + row * G_::RV + (F32 ? vg : swz_piece<G_::RV>(row, vg)) * VEC) = v[it];
        }
    }
};

// Owned state tiles: wave w owns key-sum tiles jt = w + NWAVE*m and the state
// tiles (jt, ct) of one value-column tile ct = w % CT, key tiles
// jt = m * (NWAVE / CT) + w / CT (so a wave reuses one V fragment).
template <int JT, int CT>
__device__ __forceinline__ int own_ct(int w) { return w % CT; }
template <int JT, int CT>
__device__ __forceinline__ int own_jt(int w, int m) { return m * (NWAVE / CT) + w / CT; }

// Z += phi(K_c)^T V_c on the owned tiles, S += phi(K_c)^T 1 on the owned
// key-sum tiles (the all-ones operand leaves S_j in the lanes of row j).
template <bool F32, int D, int DV, int C>
__device__ __forceinline__ void state_update(const typename Geo<F32, D, DV, C>::E *st, int w, int r, int g,
                                             f32x4 *Zown, f32x4 *Sown)
{
    typedef Geo<F32, D, DV, C> G_;
    constexpr int JT = G_::JT, CT = G_::CT;
    const int ct = own_ct<JT, CT>(w);
    if (F32) {
        const float *k = reinterpret_cast<const float *>(st) + G_::OK;
        const float *v = reinterpret_cast<const float *>(st) + G_::OV;
        const f32x4 ones = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int sa = 0; sa < G_::TBN; ++sa) {
            const f32x4 vb = trf(v, G_::RV, 16 * sa, 16 * ct, r, g);
#pragma unroll
            for (int m = 0; m < G_::ZT; ++m)
                Zown[m] = mma1(Zown[m], trf(k, G_::RK, 16 * sa, 16 * own_jt<JT, CT>(w, m), r, g), vb);
#pragma unroll
            for (int m = 0; m < G_::SMAX; ++m) {
                const int jt = w + NWAVE * m;
                if (jt < JT) Sown[m] = mma1(Sown[m], trf(k, G_::RK, 16 * sa, 16 * jt, r, g), ones);
            }
        }
    } else {
        const bf16 *kh = reinterpret_cast<const bf16 *>(st) + G_::OK;
        const bf16 *kl = reinterpret_cast<const bf16 *>(st) + G_::OKL;
        const bf16 *v = reinterpret_cast<const bf16 *>(st) + G_::OV;
        const bf16 one = (bf16)1.f;
        const bf16x8 ones = {one, one, one, one, one, one, one, one};
#pragma unroll
        for (int sa = 0; sa < G_::TBN; sa += 2) {
            // operands of this 32-token slice first, then the products with
            // the owned accumulators interleaved
            const bf16x8 vb = tr8<G_::RV>(v, 16 * sa, 16 * ct, r, g);
            bf16x8 kah[G_::ZT], kal[G_::ZT], ksh[G_::SMAX], ksl[G_::SMAX];
#pragma unroll
            for (int m = 0; m < G_::ZT; ++m) {
                const int jt = own_jt<JT, CT>(w, m);
                kah[m] = tr8<G_::RK>(kh, 16 * sa, 16 * jt, r, g);
                kal[m] = tr8<G_::RK>(kl, 16 * sa, 16 * jt, r, g);
            }
#pragma unroll
            for (int m = 0; m < G_::SMAX; ++m) {
                const int jt = w + NWAVE * m;
                if (jt < JT) {
                    ksh[m] = tr8<G_::RK>(kh, 16 * sa, 16 * jt, r, g);
                    ksl[m] = tr8<G_::RK>(kl, 16 * sa, 16 * jt, r, g);
                }
            }
#pragma unroll
            for (int m = 0; m < G_::ZT; ++m) Zown[m] = mma8(Zown[m], kah[m], vb);
#pragma unroll
            for (int m = 0; m < G_::SMAX; ++m)
                if (w + NWAVE * m < JT) Sown[m] = mma8(Sown[m], ksh[m], ones);
#pragma unroll
            for (int m = 0; m < G_::ZT; ++m) Zown[m] = mma8(Zown[m], kal[m], vb);
#pragma unroll
            for (int m = 0; m < G_::SMAX; ++m)
                if (w + NWAVE * m < JT) Sown[m] = mma8(Sown[m], ksl[m], ones);
        }
    }
}

// Load / store the owned tiles of a state in the [D][width] layout (row
// stride `ld`); S from / to `s` (lanes of row 0 of each lane group).
template <int JT, int CT, int ZT, int SMAX>
__device__ __forceinline__ void load_owned(const float *z, int64_t ld, const float *s, int w, int r, int g,
                                           f32x4 *Zown, f32x4 *Sown)
{
    const int ct = own_ct<JT, CT>(w);
#pragma unroll
    for (int m = 0; m < ZT; ++m) {
        const int jt = own_jt<JT, CT>(w, m);
#pragma unroll
        for (int i = 0; i < 4; ++i)
            Zown[m][i] = z ? z[(int64_t)(16 * jt + 4 * g + i) * ld + 16 * ct + r] : 0.f;
    }
#pragma unroll
    for (int m = 0; m < SMAX; ++m) {
        const int jt = w + NWAVE * m;
#pragma unroll
        for (int i = 0; i < 4; ++i) Sown[m][i] = (s && jt < JT) ? s[16 * jt + 4 * g + i] : 0.f;
    }
}

template <int JT, int CT, int ZT, int SMAX>
__device__ __forceinline__ void store_owned(float *z, int64_t ld, float *s, int w, int r, int g,
                                            const f32x4 *Zown, const f32x4 *Sown)
{
    const int ct = own_ct<JT, CT>(w);
    if (z) {
#pragma unroll
        for (int m = 0; m < ZT; ++m) {
            const int jt = own_jt<JT, CT>(w, m);
#pragma unroll
            for (int i = 0; i < 4; ++i) z[(int64_t)(16 * jt + 4 * g + i) * ld + 16 * ct + r] = Zown[m][i];
        }
    }
    if (s && r == 0) {
#pragma unroll
        for (int m = 0; m < SMAX; ++m) {
            const int jt = w + NWAVE * m;
            if (jt < JT) *reinterpret_cast<f32x4 *>(s + 16 * jt + 4 * g) = Sown[m];
        }
    }
}

// Publish the owned tiles to LDS: Z^T [col][dim] as MFMA A operands (hi + lo
// for bf16), and S as row DV of the same array, so that the inter-chunk
// product also yields phi(q) . S (the normaliser) in its extra row tile.
template <bool F32, int D, int DV, int C>
__device__ __forceinline__ void publish_state(typename Geo<F32, D, DV, C>::E *sm, int w, int r, int g,
                                              const f32x4 *Zown, const f32x4 *Sown)
{
    typedef Geo<F32, D, DV, C> G_;
    constexpr int JT = G_::JT, CT = G_::CT;
    const int ct = own_ct<JT, CT>(w);
    auto put = [&](int o, f32x4 x) {
        if (F32) {
            *reinterpret_cast<f32x4 *>(sm + G_::OZ + o) = x;
        } else {
            uint2 hi, lo;
            { const uint2 sp_ = split_pk(x[0], x[1]); hi.x = sp_.x; lo.x = sp_.y; }
            { const uint2 sp_ = split_pk(x[2], x[3]); hi.y = sp_.x; lo.y = sp_.y; }
            *reinterpret_cast<uint2 *>(sm + G_::OZ + o) = hi;
            *reinterpret_cast<uint2 *>(sm + G_::OZL + o) = lo;
        }
    };
#pragma unroll
    for (int m = 0; m < G_::ZT; ++m) put((16 * ct + r) * G_::RZ + 16 * own_jt<JT, CT>(w, m) + 4 * g, Zown[m]);
    if (r == 0) {
#pragma unroll
        for (int m = 0; m < G_::SMAX; ++m) {
            const int jt = w + NWAVE * m;
            if (jt < JT) put(DV * G_::RZ + 16 * jt + 4 * g, Sown[m]);
        }
    }
}

template <int I> struct IC { static constexpr int value = I; };

// f(IC<0>{}), ..., f(IC<N-1>{}): a loop whose index is a compile-time constant
template <int N, int I = 0, class F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(IC<I>{});
        static_for<N, I + 1>(f);
    }
}

// ------------------------------------------------------------------ kernels
// Partial state of one token group: A_g = phi(K_g)^T V_g (column block p),
// S_g = sum phi(k).  Written to slot `slot0 + g`.  Chunk c+2 is loaded while
// chunk c is processed.
template <bool F32, int D, int DV, int C>
__global__ void __launch_bounds__(NTHR) k_group_state(const Args a)
{
    typedef Geo<F32, D, DV, C> G_;
    typedef typename G_::E E;
    __shared__ __attribute__((aligned(16))) char smem_raw[G_::LDS_BYTES];
    E *st = reinterpret_cast<E *>(smem_raw);
    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);   // wave-uniform
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int p = wg % a.P, rest = wg / a.P, grp = rest % a.G, bh = rest / a.G;
    const int b = bh / a.H, h = bh % a.H;
    const int t_begin = grp * a.L, t_end = min(t_begin + a.L, a.N);
    constexpr int ES = F32 ? 4 : 2;
    const RowView kv{(const char *)a.k + (b * a.skb + h * a.skh) * ES, a.skn * ES, (a.N - 1) * a.skn * ES + D * ES};
    const RowView vv{(const char *)a.v + (b * a.svb + h * a.svh + p * DV) * ES, a.svn * ES,
                     (a.N - 1) * a.svn * ES + DV * ES};
    uint32_t ko[G_::NK], vo[G_::NV];
    KVRegs<F32, D, DV, C>::offsets(ko, vo, tid, kv.rs, vv.rs);

    f32x4 Zown[G_::ZT], Sown[G_::SMAX];
#pragma unroll
    for (int m = 0; m < G_::ZT; ++m) Zown[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < G_::SMAX; ++m) Sown[m] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // Every memory access is issued unconditionally (chunks past the group
    // read an empty resource), so the compiler can count outstanding accesses
    // and wait only for the chunk it is about to use.
    KVRegs<F32, D, DV, C> R[2];
    const int nch = (t_end - t_begin + C - 1) / C;
    auto issue = [&](int ch, auto slot) {
        const int t0 = t_begin + ch * C;
        const bool live = ch < nch;
        R[decltype(slot)::value].load(kv.at(t0, live), vv.at(t0, live), ko, vo);
    };
    auto step = [&](int ch, auto slot) {
        const int t0 = t_begin + ch * C;
        R[decltype(slot)::value].fill(tid, st, max(0, min(C, t_end - t0)));
        __syncthreads();
        issue(ch + 2, slot);
        state_update<F32, D, DV, C>(st, w, r, g, Zown, Sown);
        __syncthreads();
    };
    issue(0, IC<0>{});
    issue(1, IC<1>{});
    for (int ch = 0; ch < nch; ch += 2) {   // an odd count runs one empty step
        step(ch, IC<0>{});
        step(ch + 1, IC<1>{});
    }
    constexpr int SL = Slot<D, DV>::SIZE;
    float *slot = a.part + ((int64_t)(bh * a.P + p) * a.NS + a.slot0 + grp) * SL;
    store_owned<G_::JT, G_::CT, G_::ZT, G_::SMAX>(slot, DV, slot + Slot<D, DV>::Z, w, r, g, Zown, Sown);
}

// Element-wise pass over the slots of each (head, column block), all in the
// [D][DV] + [D] layout (coalesced), summing in slot order:
//  mode 0 (scan):  slot 0 <- carried-in state (or 0); slot i <- slot i-1 + slot i
//                  for i < nslots: the starting states of the token groups.
//  mode 1 (total): z_out/s_out <- carried-in state + sum of the nslots slots.
//  mode 2 (fin):   fin <- sum of the nslots slots.
//  mode 3 (memory): fin <- carried-in state (or 0), the memory that every
//                  query reads; z_out/s_out <- carried-in state + sum of the
//                  nslots slots.
// Each element is read and written by one thread, so z_out may be z_in (the
// S elements: by the thread of column block 0 only, which in mode 3 also
// writes fin's copy of S for every column block).
template <int D, int DV>
__global__ void __launch_bounds__(256) k_slots(const Args a, int nslots, int mode)
{
    constexpr int SL = Slot<D, DV>::SIZE, SZ = Slot<D, DV>::Z;
    const int hp = blockIdx.y;  // head * P + p
    const int bh = hp / a.P, p = hp % a.P;
    const int kk = blockIdx.x * 256 + threadIdx.x;
    if (kk >= SL) return;
    const bool is_s = kk >= SZ;
    if (is_s && p != 0 && (mode == 1 || mode == 3)) return;  // S is identical in every column block
    int64_t gidx;
    if (!is_s) {
        const int j = kk / DV, c = kk % DV;
        gidx = (int64_t)bh * D * D + (int64_t)j * D + p * DV + c;
    } else {
        gidx = (int64_t)bh * D + (kk - SZ);
    }
    float *src = a.part + (int64_t)hp * a.NS * SL + kk;
    float acc = 0.f;
    if (mode != 2) {
        const float *init = is_s ? a.s_in : a.z_in;
        acc = init ? init[gidx] : 0.f;
    }
    if (mode == 0) {
        // loads are batched ahead of the stores (which may alias them)
        src[0] = acc;
        for (int i0 = 1; i0 < nslots; i0 += 8) {
            const int n = min(8, nslots - i0);
            float vals[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) vals[u] = u < n ? src[(int64_t)(i0 + u) * SL] : 0.f;
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (u < n) {
                    acc += vals[u];
                    src[(int64_t)(i0 + u) * SL] = acc;
                }
            }
        }
        return;
    }
    if (mode == 3 && a.fin) {
        if (is_s) {
            for (int pp = 0; pp < a.P; ++pp) a.fin[((int64_t)bh * a.P + pp) * SL + kk] = acc;
        } else {
            a.fin[(int64_t)hp * SL + kk] = acc;
        }
    }
    float vals[8];
    int i = 0;
    for (; i + 8 <= nslots; i += 8) {
#pragma unroll
        for (int u = 0; u < 8; ++u) vals[u] = src[(int64_t)(i + u) * SL];
#pragma unroll
        for (int u = 0; u < 8; ++u) acc += vals[u];
    }
    for (; i < nslots; ++i) acc += src[(int64_t)i * SL];
    if (mode == 1 || mode == 3) {
        float *dst = is_s ? a.s_out : a.z_out;
        if (dst) dst[gidx] = acc;
    } else {
        a.fin[(int64_t)hp * SL + kk] = acc;
    }
}

// ---- device-coherent slot traffic between workgroups of one call.  The
// slots and flags are read and written with the sc0 sc1 cache policy (what
// device-scope atomics use on gfx950), so a value stored by a workgroup on one
// XCD is seen by a workgroup on another XCD without flushing any cache.
constexpr int CPOL_DEVICE = 1 | 16;   // sc0 | sc1
constexpr int CPOL_XCD = 1;            // sc0: past the CU's L1, served by the XCD's L2
__device__ __forceinline__ void dstore16(rsrc_t r, uint32_t off, f32x4 v)
{
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, off, 0, CPOL_DEVICE);
}
template <int CPOL>
__device__ __forceinline__ f32x4 dload16(rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CPOL));
}
// Index of the XCD (and so of the L2) the calling wave runs on.
__device__ __forceinline__ unsigned xcc_id()
{
    unsigned x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return x & 0xfu;
}

// Slot of one (head, column block, token group) in the single-pass kernel:
// the Z tiles as the lanes hold them (lane-contiguous 16-byte pieces, so a
// wave moves 1 KB per instruction), then S [D].
template <int D, int DV> struct FSlot {
    static constexpr int ZT = (D / 16) * (DV / 16) / NWAVE;
    static constexpr int ZF = D * DV;                 // floats of Z
    static constexpr int BYTES = (ZF + D) * 4;
    __device__ static uint32_t zoff(int w, int m, int lane) { return (uint32_t)(((w * ZT + m) * WAVE + lane) * 16); }
    __device__ static uint32_t soff(int jt, int g) { return (uint32_t)((ZF + 16 * jt + 4 * g) * 4); }
};

// Spin limit of a flag wait (a poll is a memory round trip plus a short
// sleep): a call whose flags never arrive (a bug, or memory not meant for
// this call) ends instead of hanging.
constexpr int SPIN_LIMIT = 1 << 20;

// A flag holds the call's tag (low 4 bits zero) plus the XCD index of the
// workgroup that set it.  Wait until base[i * stride] carries `tag` for
// i < n (lane i watches entry i, in rounds of 64 entries), at most
// `spin_limit` polls per round.  Returns whether all of them were set on XCD
// `xcc`; `ok` is false if the wait gave up.  Every lane of the wave runs
// this, and the results are wave-uniform.
__device__ __forceinline__ bool wait_flags(const unsigned long long *base, int stride, int n,
                                           unsigned long long tag, unsigned xcc, int lane, int spin_limit,
                                           bool &ok)
{
    bool local = true;
    ok = true;
    for (int i0 = 0; i0 < n; i0 += WAVE) {
        const int i = i0 + lane;
        const unsigned long long *f = base + (int64_t)(i < n ? i : 0) * stride;
        unsigned long long v = 0;
        bool seen = false;
        for (int spin = 0; spin < spin_limit; ++spin) {
            v = __hip_atomic_load(f, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__all(i >= n || (v & ~0xfull) == tag)) { seen = true; break; }
            __builtin_amdgcn_s_sleep(2);
        }
        ok = ok && seen;
        local = local && __all(i >= n || (v & 0xfull) == xcc);
    }
    return local;
}

// A wait that gave up: one lane of the wave counts it in the workspace's
// counter (a vector atomic), and the caller poisons what it was summing.
__device__ __forceinline__ void count_giveup(unsigned *ctr, int lane)
{
    if (lane == 0) __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The causal forward of one token group in a single pass (modes 3 and 4 of
// "How to accelerate causal linear attention" fused):
//  A. the group's own partial state A_g = phi(K_g)^T V_g, S_g = sum phi(k)
//     (group 0 adds the carried-in state), published to the group's slot
//     unless the group is the last one;
//  B. its starting state: the carried-in state (group 0) or the sum of the
//     published slots of all earlier groups of the same (head, column block);
//  C. the chunk loop (mode 3): out_t = [phi(q_t) Z_prev + sum_{s<=t in chunk}
//     P_ts v_s] / [phi(q_t) . S_prev + sum_{s<=t in chunk} P_ts + eps],
//     P = phi(Q_c) phi(K_c)^T, then Z += phi(K_c)^T V_c, S += phi(K_c)^T 1 on
//     the owned state tiles, published to LDS for the next chunk; the last
//     group writes z_out/s_out.
// MODE_APPLY (non-causal): out_t = phi(q_t) Z / (phi(q_t) . S + eps) with the
// reduced global state.
// Waiting in B is only on groups with lower workgroup indices of the same XCD
// (the logical index order is the dispatch order within an XCD), so the
// groups a workgroup waits for have been dispatched before it.
// The normaliser comes out of the same MFMAs as the numerator: S is an extra
// row of Z^T and an all-ones row is an extra row of V^T, so an extra 16-row
// output tile (whose other rows are zero operands) accumulates
// phi(q_t) . S_prev + sum_s P_ts in its first row.
constexpr int MODE_OUT = 0, MODE_APPLY = 2;

// CPG > 0 (MODE_OUT only): the group has at most CPG chunks, and all of its
// q, k, v loads are issued at the start into registers; steps A and C then
// run without waiting for memory, and the chunk loop issues stores only.
// CPG = 0: loads are streamed one chunk ahead.
template <bool F32, int D, int DV, int C, int MODE, int CPG>
__global__ void __launch_bounds__(NTHR, CPG > 0 ? res_minwg(F32, D) : minwg_of(F32, D, C)) k_chunk_fwd(const Args a)
{
    typedef Geo<F32, D, DV, C> G_;
    typedef typename G_::E E;
    typedef FSlot<D, DV> FS;
    constexpr int JT = G_::JT, CT = G_::CT, TBN = G_::TBN, BPW = G_::BPW, NQV = G_::NQV;
    constexpr int DEPTH = G_::DEPTH;
    constexpr int ES = F32 ? 4 : 2;
    constexpr int SL = Slot<D, DV>::SIZE;
    constexpr bool CAUSAL = MODE != MODE_APPLY;
    constexpr bool RES = CPG > 0;
    constexpr int NR = RES ? CPG : DEPTH;   // chunk register sets
    static_assert(!RES || MODE == MODE_OUT, "resident chunks: causal with output only");
    typedef typename pick<F32, f32x4, bf16x8>::type QOp;   // one MFMA operand of phi(q)
    __shared__ __attribute__((aligned(16))) char smem_raw[G_::LDS_BYTES];
    E *sm = reinterpret_cast<E *>(smem_raw);

    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);   // wave-uniform
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int p = wg % a.P, rest = wg / a.P, grp = rest % a.G, bh = rest / a.G;
    const int b = bh / a.H, h = bh % a.H;
    const int hp = bh * a.P + p;
    const int t_begin = grp * a.L, t_end = min(t_begin + a.L, a.N);
    const RowView qv{(const char *)a.q + (b * a.sqb + h * a.sqh) * ES, a.sqn * ES, (a.N - 1) * a.sqn * ES + D * ES};
    const RowView kv{(const char *)a.k + (b * a.skb + h * a.skh) * ES, a.skn * ES, (a.N - 1) * a.skn * ES + D * ES};
    const RowView vv{(const char *)a.v + (b * a.svb + h * a.svh + p * DV) * ES, a.svn * ES,
                     (a.N - 1) * a.svn * ES + DV * ES};
    const RowView ov{(const char *)(a.out + b * a.sob + h * a.soh + p * DV), a.son * 4, (a.N - 1) * a.son * 4 + DV * 4};
    int tbs[BPW];
    tbs[0] = w;
    if (BPW == 2) tbs[BPW - 1] = TBN - 1 - w;
    uint32_t ko[G_::NK], vo[G_::NV], qo[BPW][NQV], oo[BPW];
    if (CAUSAL) KVRegs<F32, D, DV, C>::offsets(ko, vo, tid, kv.rs, vv.rs);
#pragma unroll
    for (int bi = 0; bi < BPW; ++bi) {
        QRegs<F32, D>::offsets(qo[bi], 16 * tbs[bi] + r, qv.rs, g);
        oo[bi] = (uint32_t)((16 * tbs[bi] + r) * ov.rs + 16 * g);
    }
    const int nch = (t_end - t_begin + C - 1) / C;

    f32x4 Zown[G_::ZT], Sown[G_::SMAX];
    auto zero_state = [&]() {
#pragma unroll
        for (int m = 0; m < G_::ZT; ++m) Zown[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < G_::SMAX; ++m) Sown[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
    };

    // chunk registers and loads
    KVRegs<F32, D, DV, C> R[NR];
    QRegs<F32, D> Q[NR][BPW];
    // Every memory access is issued unconditionally (chunks past the group
    // read an empty resource; stores of rows outside the group use an
    // out-of-range offset), so the compiler can count outstanding accesses
    // and wait only for the chunk it is about to use.
    auto issue_kv = [&](int ch, auto slot) {
        const int t0 = t_begin + ch * C;
        if (CAUSAL) R[decltype(slot)::value].load(kv.at(t0, ch < nch), vv.at(t0, ch < nch), ko, vo);
    };
    auto issue_q = [&](int ch, auto slot) {
        const rsrc_t qr = qv.at(t_begin + ch * C, ch < nch);
#pragma unroll
        for (int bi = 0; bi < BPW; ++bi) Q[decltype(slot)::value][bi].load(qr, qo[bi]);
    };
    auto issue = [&](int ch, auto slot) {
        issue_kv(ch, slot);
        issue_q(ch, slot);
    };

    // ---- slot helpers: add the published slots of groups 0..n-1 of this
    // (head, column block); write z_out / s_out from (Zown, Sown)
    // (slots written on this workgroup's XCD are read from its L2; others
    // from memory)
    const unsigned my_xcc = xcc_id();
    auto add_slots = [&](int n) {
        bool ok;
        const bool local = wait_flags(a.flags + (int64_t)hp * a.G, 1, n, a.wait_tag, my_xcc, lane, a.spin_limit, ok);
        constexpr int LB = (G_::ZT + G_::SMAX) <= 5 ? 4 : 2;   // slots in flight
        const char *base = (const char *)a.part + (size_t)hp * a.G * FS::BYTES;
        auto sum = [&](auto cpol) {
            constexpr int CP = decltype(cpol)::value;
            for (int g0 = 0; g0 < n; g0 += LB) {
                f32x4 tz[LB][G_::ZT], ts[LB][G_::SMAX];
#pragma unroll
                for (int u = 0; u < LB; ++u) {
                    const bool live = g0 + u < n;
                    const rsrc_t sr = make_rsrc(base + (size_t)(live ? g0 + u : 0) * FS::BYTES, live ? FS::BYTES : 0);
#pragma unroll
                    for (int m = 0; m < G_::ZT; ++m) tz[u][m] = dload16<CP>(sr, FS::zoff(w, m, lane));
#pragma unroll
                    for (int m = 0; m < G_::SMAX; ++m) {
                        const int jt = w + NWAVE * m;
                        ts[u][m] = dload16<CP>(sr, (r == 0 && jt < JT) ? FS::soff(jt, g) : OFF_NONE);
                    }
                }
#pragma unroll
                for (int u = 0; u < LB; ++u) {
#pragma unroll
                    for (int m = 0; m < G_::ZT; ++m) Zown[m] += tz[u][m];
#pragma unroll
                    for (int m = 0; m < G_::SMAX; ++m) Sown[m] += ts[u][m];
                }
            }
        };
        if (local) sum(IC<CPOL_XCD>{});
        else sum(IC<CPOL_DEVICE>{});
        if (!ok) {   // the earlier groups' state is unknown: poison it
            count_giveup(a.giveups, lane);
#pragma unroll
            for (int m = 0; m < G_::ZT; ++m) Zown[m] = (f32x4){NAN, NAN, NAN, NAN};
#pragma unroll
            for (int m = 0; m < G_::SMAX; ++m) Sown[m] = (f32x4){NAN, NAN, NAN, NAN};
        }
    };
    // this group's slot <- (za, sa), plus (Zown, Sown) if `add`
    auto publish_slot = [&](const f32x4 *za, const f32x4 *sa, bool add) {
        const rsrc_t sr = make_rsrc((const char *)a.part + (size_t)(hp * a.G + grp) * FS::BYTES, FS::BYTES);
#pragma unroll
        for (int m = 0; m < G_::ZT; ++m) dstore16(sr, FS::zoff(w, m, lane), add ? za[m] + Zown[m] : za[m]);
#pragma unroll
        for (int m = 0; m < G_::SMAX; ++m) {
            const int jt = w + NWAVE * m;
            dstore16(sr, (r == 0 && jt < JT) ? FS::soff(jt, g) : OFF_NONE, add ? sa[m] + Sown[m] : sa[m]);
        }
    };
    // all of the workgroup's memory accesses so far are complete, then the flag
    auto set_flag = [&]() {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (tid == 0)
            __hip_atomic_store(a.flags + (int64_t)hp * a.G + grp, a.epoch | my_xcc, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    };
    auto store_final = [&]() {
        // s_out is written by the last column block; with in-place states it
        // first waits until group 0 of every column block has read s_in
        const bool s_writer = p == a.P - 1;
        bool s_ok = true;
        if (a.wait_s && s_writer) {
            (void)wait_flags(a.flags + (int64_t)bh * a.P * a.G, a.G, a.P, a.wait_tag, my_xcc, lane, a.spin_limit, s_ok);
            if (!s_ok) count_giveup(a.giveups, lane);
        }
        if (!s_ok) {   // s_in may not have been read yet: poison s_out
#pragma unroll
            for (int m = 0; m < G_::SMAX; ++m) Sown[m] = (f32x4){NAN, NAN, NAN, NAN};
        }
        store_owned<JT, CT, G_::ZT, G_::SMAX>(a.z_out ? a.z_out + (int64_t)bh * D * D + p * DV : nullptr, D,
                                              (a.s_out && s_writer) ? a.s_out + (int64_t)bh * D : nullptr,
                                              w, r, g, Zown, Sown);
    };

    // ---- per-chunk pieces of the output
    // all-ones row of V^T (lane row 0 of the extra tile), a constant operand
    QOp ones_row;
    {
        const float one = r == 0 ? 1.f : 0.f;
        if (F32) {
            f32x4 o4 = {one, one, one, one};
            ones_row = *reinterpret_cast<QOp *>(&o4);
        } else {
            const bf16 ob = (bf16)one;
            bf16x8 o8 = {ob, ob, ob, ob, ob, ob, ob, ob};
            ones_row = *reinterpret_cast<QOp *>(&o8);
        }
    }
    // phi(q) of one query tile as MFMA operands (bf16: hi + lo).  No mask is
    // needed: a query row feeds only its own output row, which is not stored
    // past the end.
    auto phi_q = [&](const QRegs<F32, D> &qr, QOp *qh, QOp *ql) {
#pragma unroll
        for (int u = 0; u < NQV; ++u) {
            float f[Vec<F32>::N];
            Vec<F32>::to_float(qr.raw[u], f);
#pragma unroll
            for (int e = 0; e < Vec<F32>::N; ++e) f[e] = phi<F32>(f[e]);
            if (F32) {
                f32x4 x = {f[0], f[1], f[2], f[3]};
                qh[u] = *reinterpret_cast<QOp *>(&x);
            } else {
                u32x4 hi, lo;
#pragma unroll
                for (int e = 0; e < 4; ++e) { const uint2 sp_ = split_pk(f[2 * e], f[2 * e + 1]); hi[e] = sp_.x; lo[e] = sp_.y; }
                qh[u] = __builtin_bit_cast(QOp, hi);
                ql[u] = __builtin_bit_cast(QOp, lo);
            }
        }
    };
    // o += phi(Q_tile) Z_shared (Z^T and S from LDS): the value tiles and, in
    // the extra tile, phi(q) . S
    // (In the extra tile every lane reads the S row: all 16 rows of that tile
    // then hold phi(q) . S, and row 0, the one that is read, also collects
    // the row sums of P.)
    auto inter = [&](f32x4 *o, const QOp *qh, const QOp *ql) {
        if (F32) {
            const float *zf = reinterpret_cast<const float *>(sm) + G_::OZ;
#pragma unroll
            for (int ct = 0; ct <= CT; ++ct)
#pragma unroll
                for (int u = 0; u < NQV; ++u) {
                    const f32x4 za = nat4(zf + (ct < CT ? 16 * ct + r : DV) * G_::RZ + 16 * u + 4 * g);
                    o[ct] = mma1(o[ct], za, *reinterpret_cast<const f32x4 *>(&qh[u]));
                }
        } else {
            const bf16 *zh = reinterpret_cast<const bf16 *>(sm) + G_::OZ;
            const bf16 *zl = reinterpret_cast<const bf16 *>(sm) + G_::OZL;
            // all operands first, then the products with the CT + 1
            // accumulators interleaved (independent MFMA chains)
            bf16x8 a_hi[CT + 1][NQV], a_lo[CT + 1][NQV];
#pragma unroll
            for (int ct = 0; ct <= CT; ++ct) {
                const int zo = (ct < CT ? 16 * ct + r : DV) * G_::RZ + 8 * g;
#pragma unroll
                for (int u = 0; u < NQV; ++u) { a_hi[ct][u] = nat8(zh + zo + 32 * u); a_lo[ct][u] = nat8(zl + zo + 32 * u); }
            }
#pragma unroll
            for (int u = 0; u < NQV; ++u) {
                const bf16x8 qh8 = *reinterpret_cast<const bf16x8 *>(&qh[u]);
                const bf16x8 ql8 = *reinterpret_cast<const bf16x8 *>(&ql[u]);
#pragma unroll
                for (int ct = 0; ct <= CT; ++ct) o[ct] = mma8(o[ct], a_hi[ct][u], qh8);
#pragma unroll
                for (int ct = 0; ct <= CT; ++ct) o[ct] = mma8(o[ct], a_lo[ct][u], qh8);
#pragma unroll
                for (int ct = 0; ct <= CT; ++ct) o[ct] = mma8(o[ct], a_hi[ct][u], ql8);
            }
        }
    };
    // o += intra-chunk term of query tile tb over key tiles sa <= tb: scores
    // P^T (rows = keys, columns = queries) feed P V as the B operand directly;
    // the extra tile gets the row sums of P
    auto intra = [&](f32x4 *o, const QOp *qh, int tb) {
        if (F32) {
            const float *kf = reinterpret_cast<const float *>(sm) + G_::OK;
            const float *vf = reinterpret_cast<const float *>(sm) + G_::OV;
            for (int sa = 0; sa <= tb; ++sa) {
                f32x4 pt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < NQV; ++u)
                    pt = mma1(pt, nat4(kf + (16 * sa + r) * G_::RK + 16 * u + 4 * g), *reinterpret_cast<const f32x4 *>(&qh[u]));
                if (sa == tb) {
#pragma unroll
                    for (int i = 0; i < 4; ++i) if (4 * g + i > r) pt[i] = 0.f;
                }
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) o[ct] = mma1(o[ct], trf(vf, G_::RV, 16 * sa, 16 * ct, r, g), pt);
                o[CT] = mma1(o[CT], *reinterpret_cast<const f32x4 *>(&ones_row), pt);
            }
        } else {
            const bf16 *kb = reinterpret_cast<const bf16 *>(sm) + G_::OK;
            const bf16 *vb = reinterpret_cast<const bf16 *>(sm) + G_::OV;
            const bf16 zr = (bf16)0.f;
            const bf16x8 ones8 = *reinterpret_cast<const bf16x8 *>(&ones_row);
            for (int sa = 0; sa <= tb; sa += 2) {
                const bool two = sa + 1 <= tb;
                f32x4 pt0 = {0.f, 0.f, 0.f, 0.f}, pt1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int u = 0; u < NQV; ++u) {
                    const bf16x8 qh8 = *reinterpret_cast<const bf16x8 *>(&qh[u]);
                    pt0 = mma8(pt0, nat8(kb + swz<G_::RK>(16 * sa + r, 32 * u + 8 * g)), qh8);
                    if (two) pt1 = mma8(pt1, nat8(kb + swz<G_::RK>(16 * sa + 16 + r, 32 * u + 8 * g)), qh8);
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
                u32x4 phw = {0u, 0u, 0u, 0u}, plw = {0u, 0u, 0u, 0u};
                { const uint2 sp_ = split_pk(pt0[0], pt0[1]); phw[0] = sp_.x; plw[0] = sp_.y; }
                { const uint2 sp_ = split_pk(pt0[2], pt0[3]); phw[1] = sp_.x; plw[1] = sp_.y; }
                if (two) {
                    { const uint2 sp_ = split_pk(pt1[0], pt1[1]); phw[2] = sp_.x; plw[2] = sp_.y; }
                    { const uint2 sp_ = split_pk(pt1[2], pt1[3]); phw[3] = sp_.x; plw[3] = sp_.y; }
                }
                const bf16x8 bh8 = __builtin_bit_cast(bf16x8, phw);
                const bf16x8 bl8 = __builtin_bit_cast(bf16x8, plw);
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) {
                    bf16x4 va0 = tr4<G_::RV>(vb, 16 * sa, 16 * ct, r, g);
                    bf16x4 va1 = {zr, zr, zr, zr};
                    if (two) va1 = tr4<G_::RV>(vb, 16 * sa + 16, 16 * ct, r, g);
                    const bf16x8 a8 = __builtin_shufflevector(va0, va1, 0, 1, 2, 3, 4, 5, 6, 7);
                    o[ct] = mma8(o[ct], a8, bh8);
                    o[ct] = mma8(o[ct], a8, bl8);
                }
                o[CT] = mma8(o[CT], ones8, bh8);
                o[CT] = mma8(o[CT], ones8, bl8);
            }
        }
    };
    // out rows of query tile tb in chunk ch = value tiles / (normaliser + eps)
    auto finish = [&](const f32x4 *o, int ch, int tb) {
        const int t0 = t_begin + ch * C;
        const int nval = min(C, t_end - t0);
        const int tq = 16 * tb + r;
        // normaliser of query r: row 0 of the extra tile, held by lane r
        const float den = __shfl(o[CT][0], r) + a.eps;
        const float inv = a.unnorm ? 1.f : __builtin_amdgcn_rcpf(den);   // within 1 ulp
        const rsrc_t orr = ov.at(t0);
        const uint32_t obase = tq < nval ? (uint32_t)(tq * ov.rs + 16 * g) : OFF_NONE;
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) bstore16(orr, tq < nval ? obase + 64 * ct : OFF_NONE, o[ct] * inv);
    };
    auto zero_o = [&](f32x4 *o) {
#pragma unroll
        for (int ct = 0; ct <= CT; ++ct) o[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
    };

    // ---- one chunk of the streaming loop (and of the non-causal readout):
    // stage K, V and phi(q); the output rows; the state update
    // (resident bf16 groups: phi(K) is split into hi + lo in registers, then
    // copied to LDS; the own-state step's split is not held, register budget)
    auto step = [&](int ch, auto slot) {
        constexpr int S_ = decltype(slot)::value;
        const int t0 = t_begin + ch * C;
        if constexpr (RES && !F32) {
            R[S_].phi_split(tid, min(C, t_end - t0));
            R[S_].stage(tid, sm);
        } else if (CAUSAL) {
            R[S_].fill(tid, sm, min(C, t_end - t0));
        }
        QOp qhi[BPW][NQV], qlo[BPW][NQV];
#pragma unroll
        for (int bi = 0; bi < BPW; ++bi) phi_q(Q[S_][bi], qhi[bi], qlo[bi]);
        if (CAUSAL || ch == 0) __syncthreads();   // stage and published state visible
        // ---- request chunk ch + DEPTH into the registers just consumed
        if constexpr (!RES) issue(ch + DEPTH, slot);
        else if constexpr (S_ + 2 < NR) issue_q(ch + 2, IC<S_ + 2>{});
#pragma unroll
        for (int bi = 0; bi < BPW; ++bi) {
            f32x4 o[CT + 1];   // value tiles, then the normaliser tile
            zero_o(o);
            inter(o, qhi[bi], qlo[bi]);
            if (CAUSAL) intra(o, qhi[bi], tbs[bi]);
            finish(o, ch, tbs[bi]);
        }
        if (CAUSAL) {
            state_update<F32, D, DV, C>(sm, w, r, g, Zown, Sown);
            __syncthreads();   // every wave is done with this chunk's stage and state
            publish_state<F32, D, DV, C>(sm, w, r, g, Zown, Sown);
        }
    };

    if constexpr (MODE == MODE_APPLY) {
        const float *sl = a.fin + (int64_t)hp * SL;
        load_owned<JT, CT, G_::ZT, G_::SMAX>(sl, DV, sl + Slot<D, DV>::Z, w, r, g, Zown, Sown);
        publish_state<F32, D, DV, C>(sm, w, r, g, Zown, Sown);
        issue(0, IC<0>{});
        for (int ch = 0; ch < nch; ++ch) step(ch, IC<0>{});
        return;
    } else {
        f32x4 Zin[G_::ZT], Sin[G_::SMAX];
        if (grp == 0) {
            load_owned<JT, CT, G_::ZT, G_::SMAX>(a.z_in ? a.z_in + (int64_t)bh * D * D + p * DV : nullptr, D,
                                                 a.s_in ? a.s_in + (int64_t)bh * D : nullptr, w, r, g, Zin, Sin);
        }
        const bool last = grp == a.G - 1;
        if constexpr (RES) {
            // ================= register-resident group: A, B, C with every load
            // of the group held in registers.  k and v stream two chunks
            // ahead through A (loads only, so the compiler waits for exactly
            // the chunk in use); q is requested after the last k and v; the
            // chunk loop C then issues stores only.
            constexpr int KV0 = CPG < 2 ? CPG : 2;   // k, v chunks requested up front
            auto issue_rest = [&]() {   // k, v of the remaining chunks
                static_for<CPG>([&](auto c) { if constexpr (c.value >= KV0) issue_kv(c.value, c); });
            };
            static_for<KV0>([&](auto c) { issue_kv(c.value, c); });
            if (!last) {
                if (grp == 0) {
#pragma unroll
                    for (int m = 0; m < G_::ZT; ++m) Zown[m] = Zin[m];
#pragma unroll
                    for (int m = 0; m < G_::SMAX; ++m) Sown[m] = Sin[m];
                } else {
                    zero_state();
                }
                static_for<CPG>([&](auto cc) {
                    constexpr int c = decltype(cc)::value;
                    // k, v of chunk c + 2 while chunk c is used
                    if constexpr (c + 2 < CPG) issue_kv(c + 2, IC<c + 2>{});
                    if (c < nch) {
                        if constexpr (F32) {
                            R[c].fill(tid, sm, min(C, t_end - (t_begin + c * C)));
                        } else {
                            R[c].phi_split(tid, min(C, t_end - (t_begin + c * C)));
                            R[c].stage(tid, sm);
                        }
                        __syncthreads();
                        state_update<F32, D, DV, C>(sm, w, r, g, Zown, Sown);
                        __syncthreads();
                    }
                });
                publish_slot(Zown, Sown, false);
                set_flag();
            } else {
                issue_rest();
                if (grp == 0 && a.wait_s) set_flag();   // only signals that z_in / s_in have been read
            }
            // q streams through the chunk loop two chunks ahead; the first two
            // are requested here, after the look-back's loads
            // ---- B: the state before the group
            if (grp == 0) {
#pragma unroll
                for (int m = 0; m < G_::ZT; ++m) Zown[m] = Zin[m];
#pragma unroll
                for (int m = 0; m < G_::SMAX; ++m) Sown[m] = Sin[m];
            } else {
                zero_state();
                add_slots(grp);
            }
            static_for<KV0>([&](auto c) { issue_q(c.value, c); });
            publish_state<F32, D, DV, C>(sm, w, r, g, Zown, Sown);
            // ---- C: the chunk loop from registers
            static_for<CPG>([&](auto c) {
                if (c.value < nch) step(c.value, c);
            });
            if (last) store_final();
            return;
        } else {
            // ================= streamed group: A, B, C as described above
            const bool publish = !last;
            if (publish) {
                if (grp == 0) {
#pragma unroll
                    for (int m = 0; m < G_::ZT; ++m) Zown[m] = Zin[m];
#pragma unroll
                    for (int m = 0; m < G_::SMAX; ++m) Sown[m] = Sin[m];
                } else {
                    zero_state();
                }
                // chunks in reverse order, so that the chunk loop's first chunks
                // are the most recently read; loads run two chunks ahead
                KVRegs<F32, D, DV, C> RA[2];
                auto issue_a = [&](int i, auto slot) {
                    const int ch = max(nch - 1 - i, 0);
                    const int t0 = t_begin + ch * C;
                    RA[decltype(slot)::value].load(kv.at(t0, i < nch), vv.at(t0, i < nch), ko, vo);
                };
                auto step_a = [&](int i, auto slot) {
                    const int t0 = t_begin + max(nch - 1 - i, 0) * C;
                    RA[decltype(slot)::value].fill(tid, sm, i < nch ? min(C, t_end - t0) : 0);
                    __syncthreads();
                    issue_a(i + 2, slot);
                    state_update<F32, D, DV, C>(sm, w, r, g, Zown, Sown);
                    __syncthreads();
                };
                issue_a(0, IC<0>{});
                issue_a(1, IC<1>{});
                for (int i = 0; i < nch; i += 2) {   // an odd count runs one empty step
                    step_a(i, IC<0>{});
                    step_a(i + 1, IC<1>{});
                }
                publish_slot(Zown, Sown, false);
            }
            // group 0 also signals that it has read z_in / s_in (in-place states)
            if (publish || (grp == 0 && a.wait_s)) set_flag();
            issue(0, IC<0>{});   // the first chunk's loads overlap the look-back
            if (grp == 0) {
#pragma unroll
                for (int m = 0; m < G_::ZT; ++m) Zown[m] = Zin[m];
#pragma unroll
                for (int m = 0; m < G_::SMAX; ++m) Sown[m] = Sin[m];
            } else {
                zero_state();
                add_slots(grp);
            }
            publish_state<F32, D, DV, C>(sm, w, r, g, Zown, Sown);
            static_assert(DEPTH == 1, "one chunk of loads in flight");
            for (int ch = 0; ch < nch; ++ch) step(ch, IC<0>{});
            if (last) store_final();
        }
    }
}

// Logical (unit = head x column block, group) of a column-split workgroup
// from its remapped index.  When the remap is active and every XCD holds
// whole units, the first half of an XCD's workgroups (dispatched first, one
// per CU) takes the first half of each unit's groups and the second half the
// rest, so a CU pairs group g with group g + G/2 of one unit rather than two
// groups g: the look-back reads, which grow with g, are spread over the CUs.
// Every group still comes after all earlier groups of its unit in dispatch
// order within the XCD.  Otherwise the plain order (column block fastest,
// then group, then head).
__device__ __forceinline__ void cs_unit_group(int wg, int n, int G, int P, int &unit, int &grp)
{
    const int nx = n >> 3;
    if ((n & 7) == 0 && G >= 2 && nx % G == 0) {
        const int x = wg / nx, i = wg % nx, ux = nx / G, gl = G / 2;
        int u, gg;
        if (i < ux * gl) {
            u = i / gl;
            gg = i % gl;
        } else {
            const int i2 = i - ux * gl;
            u = i2 / (G - gl);
            gg = gl + i2 % (G - gl);
        }
        unit = x * ux + u;
        grp = gg;
    } else {
        const int p = wg % P, rest = wg / P;
        grp = rest % G;
        unit = (rest / G) * P + p;
    }
}

// ================================================================ column-split causal kernel
// bf16 inputs, 64-token chunks, a group of at most CPG chunks per workgroup
// with every q, k, v load of the group held in registers.  Each of the 4 waves
// owns 16 of the workgroup's 64 value columns for the whole group: its slice
// of the state Z (all D key dims x 16 columns) stays in its registers, and it
// holds D / 64 of the S tiles (the S operands of the normalisers go through
// LDS).  Per chunk the 10 causal 16x16 score tiles are split over the waves
// and shared through LDS; each wave then forms the inter- and intra-chunk
// terms of its 16 columns for all 64 queries and the normaliser of one
// 16-query tile, which goes to the other waves through LDS with the next
// barrier.
//
// Precision: phi = 1 + psi with psi = elu, and only psi(q), psi(k) are bf16
// MFMA operands (exact for positive inputs; the all-ones part of phi is
// carried in fp32).  So
//   phi(q) . z     = sum_i z_i + psi(q) . z            (z a column of Z, or S)
//   phi(q) . phi(k) = d + sum psi(q) + sum psi(k) + psi(q) . psi(k)
//   Z += psi(K)^T V + 1 (column sums of V)^T,  S += psi(K)^T 1 + (tokens) 1,
// where the sums over dims of psi(k) (formed in pass 1) and psi(q) (formed in
// the stage) are fp32 sums of the values before rounding, and the sums over
// dims of Z and S are MFMA products with an all-ones operand.  The fp32
// values fed back as operands -- the scores P and the state (Z, S) -- are
// split into bf16 hi + lo.
//
// State tile layout: tile jt = 2u + hf, row m = 4g + i of the tile holds key
// dim pi(jt, m) = 32u + 8g + 4hf + i.  Then tiles 2u and 2u + 1 of a lane hold
// dims 32u + 8g .. 32u + 8g + 7 in order: the natural operand layout of a
// 32-dim contraction step, which is also how phi(q) and phi(k) rows are read.
template <int D> struct CSGeo {
    static constexpr int C = 64, DV = 64;
    static constexpr int JT = D / 16;              // state tiles (key dims) per wave
    static constexpr int KS = D / 32;              // 32-dim contraction steps
    static constexpr int VPR = D / 8;              // 16-byte vectors per q / k row
    static constexpr int NK = C * VPR / NTHR;      // k (and q) vectors per thread per chunk
    static constexpr int NV = C * (DV / 8) / NTHR; // v vectors per thread per chunk
    // LDS, bf16 elements: the stage of psi(K) [C][D] and of V [C][DV] (rows
    // swizzled, swz); the score operands [6 pairs][hi, lo][64 lanes][8]; the
    // S operands [2][hi, lo][KS][4 lane groups][8]; psi(Q) of every chunk of
    // the group [CPG][C][D] (swizzled); then fp32: the normalisers [CPG][C],
    // the per-wave sums of S [2][4], the row sums of psi(q) [2][C] and of
    // psi(k) [CPG][C].
    static constexpr int OK = 0, OV = C * D, OP = OV + C * DV, OSO = OP + 6 * 2 * 64 * 8;
    static constexpr int OQ = OSO + 2 * 2 * KS * 4 * 8;
    static constexpr int bf16_elems(int cpg) { return OQ + cpg * C * D; }
    static constexpr int lds_bytes(int cpg) { return bf16_elems(cpg) * 2 + (2 * cpg * C + 8 + 2 * C) * 4; }
    static_assert(NK * NTHR == C * VPR && NV * NTHR == C * DV / 8, "whole vectors per thread");
};
__device__ __forceinline__ int cs_dim(int jt, int m) { return 32 * (jt >> 1) + 8 * (m >> 2) + 4 * (jt & 1) + (m & 3); }

// phi(K)^T operand of state tile jt for tokens s0 + 4g .. s0 + 4g + 3: lane n
// addresses token row s0 + 4g + n/4 and the 4 dims starting at
// 32u + 8(n%4) + 4hf; the transpose read then hands lane n the dim
// cs_dim(jt, n) (element n%4 of the piece addressed by lane 4*row + n/4).
template <int W>
__device__ __forceinline__ bf16x4 cs_ktr4(const bf16 *base, int s0, int jt, int n, int g)
{
    const bf16 *p = base + swz<W>(s0 + 4 * g + (n >> 2), 32 * (jt >> 1) + 8 * (n & 3) + 4 * (jt & 1));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4 *)(bf16 *)p);
}
template <int W>
__device__ __forceinline__ bf16x8 cs_ktr8(const bf16 *base, int s0, int jt, int n, int g)
{
    const bf16x4 x = cs_ktr4<W>(base, s0, jt, n, g), y = cs_ktr4<W>(base, s0 + 16, jt, n, g);
    return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}
// bf16 hi + lo operands of two fp32 fragments (8 values in order)
__device__ __forceinline__ void cs_split(f32x4 x, f32x4 y, bf16x8 &hi, bf16x8 &lo)
{
    u32x4 h, l;
    { const uint2 s_ = split_pk(x[0], x[1]); h[0] = s_.x; l[0] = s_.y; }
    { const uint2 s_ = split_pk(x[2], x[3]); h[1] = s_.x; l[1] = s_.y; }
    { const uint2 s_ = split_pk(y[0], y[1]); h[2] = s_.x; l[2] = s_.y; }
    { const uint2 s_ = split_pk(y[2], y[3]); h[3] = s_.x; l[3] = s_.y; }
    hi = __builtin_bit_cast(bf16x8, h);
    lo = __builtin_bit_cast(bf16x8, l);
}
// psi(x) = elu(x) = phi(x) - 1: x above zero, e^x - 1 at or below it.  As
// e^x - 1 >= x everywhere, this is max(x, min(e^x, 1) - 1): four
// instructions (the min is the clamp bit of v_exp_f32; the NaN-propagating
// maximum keeps psi(NaN) = NaN; psi(-inf) = -1, psi(+inf) = +inf).
__device__ __forceinline__ float psi(float x)
{
    const float e = __builtin_amdgcn_fmed3f(__builtin_amdgcn_exp2f(x * 1.44269504088896340736f), 0.f, 1.f);
    return __builtin_elementwise_maximum(x, e - 1.f);
}
// psi of 8 packed bf16 values rounded to bf16 (nearest even); `sum` += the
// sum of the values before rounding (it enters only the scores, where the
// difference, below 2^-9 of each |psi|, is far below their split precision)
__device__ __forceinline__ u32x4 cs_psi8(u32x4 x, float &sum)
{
    float f[8];
    Vec<false>::to_float(x, f);
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float a = psi(f[2 * e]), b = psi(f[2 * e + 1]);
        y[e] = pk_bf16(a, b);
        sum += a + b;
    }
    return y;
}
__device__ __forceinline__ u32x4 cs_psi8(u32x4 x)
{
    float f[8];
    Vec<false>::to_float(x, f);
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = pk_bf16(psi(f[2 * e]), psi(f[2 * e + 1]));
    return y;
}

template <int D, int CPG, bool UNNORM>
__global__ void __launch_bounds__(NTHR, 2) k_cs_fwd(const Args a)
{
    typedef CSGeo<D> T;
    typedef FSlot<D, 64> FS;
    constexpr int C = T::C, DV = T::DV, JT = T::JT, KS = T::KS, VPR = T::VPR, NK = T::NK, NV = T::NV;
    static_assert(FS::ZT == JT, "slot tiles per wave");
    __shared__ __attribute__((aligned(16))) char smem_raw[T::lds_bytes(CPG)];
    bf16 *sm = reinterpret_cast<bf16 *>(smem_raw);
    float *den_s = reinterpret_cast<float *>(smem_raw + T::bf16_elems(CPG) * 2);   // [CPG][C]
    float *ssum_s = den_s + CPG * C;                                                // [2][4]
    float *qsum_s = ssum_s + 8;                                                     // [2][C]
    float *ksum_s = qsum_s + 2 * C;                                                 // [CPG][C]
    auto kbuf = [&]() { return sm + T::OK; };
    auto vbuf = [&]() { return sm + T::OV; };
    auto qslot = [&](int c) { return sm + T::OQ + c * C * D; };

    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);   // wave-uniform
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    int hp, grp;
    cs_unit_group(wg, gridDim.x, a.G, a.P, hp, grp);
    const int p = hp % a.P, bh = hp / a.P;
    const int b = bh / a.H, h = bh % a.H;
    const int t_begin = grp * a.L, t_end = min(t_begin + a.L, a.N);
    const int nch = (t_end - t_begin + C - 1) / C;
    const bool last = grp == a.G - 1;
    const bool s_writer = p == a.P - 1;
    const RowView qv{(const char *)a.q + (b * a.sqb + h * a.sqh) * 2, a.sqn * 2, (a.N - 1) * a.sqn * 2 + D * 2};
    const RowView kv{(const char *)a.k + (b * a.skb + h * a.skh) * 2, a.skn * 2, (a.N - 1) * a.skn * 2 + D * 2};
    const RowView vv{(const char *)a.v + (b * a.svb + h * a.svh + p * DV) * 2, a.svn * 2,
                     (a.N - 1) * a.svn * 2 + DV * 2};
    const RowView ov{(const char *)(a.out + b * a.sob + h * a.soh + p * DV), a.son * 4, (a.N - 1) * a.son * 4 + DV * 4};

    // cooperative loads: vector `it` of a thread is item tid + it * NTHR of the
    // chunk, row item / (vectors per row); q, k, v are requested two chunks
    // ahead
    uint32_t ko[NK], qo[NK], vo[NV];
#pragma unroll
    for (int it = 0; it < NK; ++it) {
        const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
        ko[it] = (uint32_t)(row * kv.rs + vec * 16);
        qo[it] = (uint32_t)(row * qv.rs + vec * 16);
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
        const int item = tid + it * NTHR;
        vo[it] = (uint32_t)((item / 8) * vv.rs + (item % 8) * 16);
    }
    u32x4 Kr[CPG][NK], Vr[CPG][NV], Qr[CPG][NK];
    auto issue_kv = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        const int t0 = t_begin + c * C;
        const rsrc_t kr = kv.at(t0, c < nch), vr = vv.at(t0, c < nch);
#pragma unroll
        for (int it = 0; it < NK; ++it) Kr[c][it] = bload16nt(kr, ko[it]);
#pragma unroll
        for (int it = 0; it < NV; ++it) Vr[c][it] = bload16nt(vr, vo[it]);
    };
    auto issue_q = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        const rsrc_t qr = qv.at(t_begin + c * C, c < nch);
#pragma unroll
        for (int it = 0; it < NK; ++it) Qr[c][it] = bload16nt(qr, qo[it]);
    };
    auto nval_of = [&](int c) { return min(C, t_end - (t_begin + c * C)); };
    // the stage of chunk c in pass 2: psi(K) (already in registers) and V
    // (one buffer each), psi(Q) into slot c, the row sums of psi(q) into
    // buffer c % 2 (those of psi(k) are in place since pass 1).
    // Rows past the end of the sequence read as zeros (outside the buffer
    // resource), and psi(0) = 0, so they add nothing to the state; the scores
    // mask those keys.
    auto stage = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        const int buf = c & 1;
        bf16 *Kb = kbuf(), *Qb = qslot(c), *Vb = vbuf();
#pragma unroll
        for (int it = 0; it < NK; ++it) {
            const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
            float qs = 0.f;
            *reinterpret_cast<u32x4 *>(Kb + swz<D>(row, vec * 8)) = Kr[c][it];
            *reinterpret_cast<u32x4 *>(Qb + swz<D>(row, vec * 8)) = cs_psi8(Qr[c][it], qs);
            // row sum over the VPR consecutive lanes of the row
#pragma unroll
            for (int m = 1; m < VPR; m <<= 1) qs += __shfl_xor(qs, m);
            if (vec == 0) qsum_s[buf * C + row] = qs;
        }
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int item = tid + it * NTHR, row = item / 8, vec = item % 8;
            *reinterpret_cast<u32x4 *>(Vb + swz<64>(row, vec * 8)) = Vr[c][it];
        }
    };
    // the stage of pass 1: k becomes psi(k) in its registers, its row sums
    // go to ksum_s[c]; psi(K) and V are staged for the state update (the
    // last group, which has no pass-1 state, stages nothing)
    auto stage_kv = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        bf16 *Kb = kbuf(), *Vb = vbuf();
#pragma unroll
        for (int it = 0; it < NK; ++it) {
            const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
            float ks = 0.f;
            Kr[c][it] = cs_psi8(Kr[c][it], ks);
#pragma unroll
            for (int m = 1; m < VPR; m <<= 1) ks += __shfl_xor(ks, m);
            if (vec == 0) ksum_s[c * C + row] = ks;
            if (!last) *reinterpret_cast<u32x4 *>(Kb + swz<D>(row, vec * 8)) = Kr[c][it];
        }
        if (!last) {
#pragma unroll
            for (int it = 0; it < NV; ++it) {
                const int item = tid + it * NTHR, row = item / 8, vec = item % 8;
                *reinterpret_cast<u32x4 *>(Vb + swz<64>(row, vec * 8)) = Vr[c][it];
            }
        }
    };

    bf16x8 ones8;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones8[e] = (bf16)1.f;
    // ---- the wave's state: Z[dims][16w + r] over all key dims, and the S
    // tiles jt = w + NWAVE m (SPW of them; every column of an S tile holds
    // S).  First the group-local running state (group 0: from the carried-in
    // state), then the state before the group (Ze, Se).
    constexpr int SPW = JT / NWAVE;
    static_assert(JT % NWAVE == 0, "S tiles split evenly over the waves");
    f32x4 Z[JT], S[SPW], Ze[JT], Se[SPW];
    auto load_state = [&](f32x4 *z4, f32x4 *s4, const float *z, const float *s) __attribute__((always_inline)) {
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) z4[jt][i] = z ? z[(int64_t)cs_dim(jt, 4 * g + i) * D + p * DV + 16 * w + r] : 0.f;
#pragma unroll
        for (int m = 0; m < SPW; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) s4[m][i] = s ? s[cs_dim(w + NWAVE * m, 4 * g + i)] : 0.f;
    };
    // hi + lo operands of a state, and its sums over the key dims (every row
    // of the result: sum_i z[i][column])
    auto state_ops = [&](const f32x4 *z4, bf16x8 *zh, bf16x8 *zl, f32x4 &zsum) __attribute__((always_inline)) {
        zsum = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            cs_split(z4[2 * u], z4[2 * u + 1], zh[u], zl[u]);
            zsum = mma8(zsum, zh[u], ones8);
            zsum = mma8(zsum, zl[u], ones8);
        }
    };
    // S operands for the normalisers, shared through LDS (the hi/lo operand
    // of a lane depends only on its lane group g): [2][hi, lo][KS][g][8];
    // every wave writes the halves of its S tiles and the sum of their values
    auto sops_at = [&](int buf, int hl, int u, int gg) { return sm + T::OSO + (((buf * 2 + hl) * KS + u) * 4 + gg) * 8; };
    auto put_sops = [&](const f32x4 *s4, int buf) __attribute__((always_inline)) {
        float part = 0.f;
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
            const int jt = w + NWAVE * m;
            uint2 hi, lo;
            { const uint2 s_ = split_pk(s4[m][0], s4[m][1]); hi.x = s_.x; lo.x = s_.y; }
            { const uint2 s_ = split_pk(s4[m][2], s4[m][3]); hi.y = s_.x; lo.y = s_.y; }
            if (r == 0) {
                *reinterpret_cast<uint2 *>(sops_at(buf, 0, jt >> 1, g) + 4 * (jt & 1)) = hi;
                *reinterpret_cast<uint2 *>(sops_at(buf, 1, jt >> 1, g) + 4 * (jt & 1)) = lo;
            }
            part += (s4[m][0] + s4[m][1]) + (s4[m][2] + s4[m][3]);
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (lane == 0) ssum_s[buf * 4 + w] = part;
    };
    // the normaliser of query tile m: sum S + S . psi(q) + (intra, by the caller)
    auto sdot = [&](int buf, const bf16x8 *qb) __attribute__((always_inline)) {
        f32x4 dn;
        const f32x4 s4 = *reinterpret_cast<const f32x4 *>(ssum_s + buf * 4);
        const float s0 = (s4[0] + s4[1]) + (s4[2] + s4[3]);
        dn = (f32x4){s0, s0, s0, s0};
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            dn = mma8(dn, nat8(sops_at(buf, 0, u, g)), qb[u]);
            dn = mma8(dn, nat8(sops_at(buf, 1, u, g)), qb[u]);
        }
        return dn;
    };
    auto q_ops = [&](const bf16 *Qb, int m, bf16x8 *qb) __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < KS; ++u) qb[u] = nat8(Qb + swz<D>(16 * m + r, 32 * u + 8 * g));
    };
    // ---- scores: tile (sa, m) of P^T (keys 16 sa.., queries 16 m..) is
    // computed by one wave, split into bf16 hi + lo and written to LDS as half
    // of the P V operand of pair (m, sa / 2): [pair][hi, lo][lane][8]
    // first pair of query tile m: 0, 1, 2, 4
    auto pbase = [](int m) { return m + (m == 3 ? 1 : 0); };
    auto pop_at = [&](int pair, int hl, int ln) { return sm + T::OP + ((pair * 2 + hl) * WAVE + ln) * 8; };
    // tiles above the diagonal that complete a pair: zero once
    if (tid < 4 * WAVE) {
        const int which = tid / WAVE, ln = tid % WAVE;   // (pair 0 | pair 3) x (hi | lo)
        *reinterpret_cast<uint2 *>(pop_at(which < 2 ? 0 : 3, which & 1, ln) + 4) = make_uint2(0u, 0u);
    }
    auto score_tile = [&](const bf16x8 *ka, const bf16x8 *qb, int sa, int m, int nv, int buf, int kc) __attribute__((always_inline)) {
        // d + sum psi(q_t) + sum psi(k_s) (row sums from the stage), then
        // + psi(k_s) . psi(q_t)
        f32x4 pt = *reinterpret_cast<const f32x4 *>(ksum_s + kc * C + 16 * sa + 4 * g) +
                   ((float)D + qsum_s[buf * C + 16 * m + r]);
#pragma unroll
        for (int u = 0; u < KS; ++u) pt = mma8(pt, ka[u], qb[u]);
        // causal mask inside the diagonal tile (key 4g + i > query r) and keys
        // past the end of a ragged chunk (selects, no branches)
        const int lim = min(sa == m ? r - 4 * g : 3, nv - 1 - 16 * sa - 4 * g);   // last kept i
#pragma unroll
        for (int i = 0; i < 4; ++i) pt[i] = i <= lim ? pt[i] : 0.f;
        uint2 hi, lo;
        { const uint2 s_ = split_pk(pt[0], pt[1]); hi.x = s_.x; lo.x = s_.y; }
        { const uint2 s_ = split_pk(pt[2], pt[3]); hi.y = s_.x; lo.y = s_.y; }
        const int pair = pbase(m) + sa / 2, half = sa & 1;
        *reinterpret_cast<uint2 *>(pop_at(pair, 0, lane) + 4 * half) = hi;
        *reinterpret_cast<uint2 *>(pop_at(pair, 1, lane) + 4 * half) = lo;
    };

    // state update from the stage of one chunk: Z += psi(K)^T V + 1 (column
    // sums of V)^T, the wave's S tiles += psi(K)^T 1 + nv (va: V operands)
    auto update_state = [&](const bf16 *Kb, const bf16x8 *va, int nv) __attribute__((always_inline)) {
        f32x4 cv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) cv = mma8(cv, ones8, va[sg]);
        const float fn = (float)nv;
        constexpr int JR = JT <= 4 ? JT : 2;   // state tiles whose operands are read together
#pragma unroll
        for (int j0 = 0; j0 < JT; j0 += JR) {
            bf16x8 kt[JR][2];
#pragma unroll
            for (int j = 0; j < JR; ++j)
#pragma unroll
                for (int sg = 0; sg < 2; ++sg) kt[j][sg] = cs_ktr8<D>(Kb, 32 * sg, j0 + j, r, g);
#pragma unroll
            for (int j = 0; j < JR; ++j) {
#pragma unroll
                for (int sg = 0; sg < 2; ++sg) Z[j0 + j] = mma8(Z[j0 + j], kt[j][sg], va[sg]);
                Z[j0 + j] += cv;
            }
        }
#pragma unroll
        for (int m = 0; m < SPW; ++m) {
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) S[m] = mma8(S[m], cs_ktr8<D>(Kb, 32 * sg, w + NWAVE * m, r, g), ones8);
            S[m] += (f32x4){fn, fn, fn, fn};
        }
    };
    auto load_start = [&]() __attribute__((always_inline)) {   // the state at the start of the group (group 0: carried in)
        if (grp == 0) load_state(Z, S, a.z_in ? a.z_in + (int64_t)bh * D * D : nullptr, a.s_in ? a.s_in + (int64_t)bh * D : nullptr);
        else load_state(Z, S, nullptr, nullptr);
    };

    const unsigned my_xcc = xcc_id();
    constexpr bool EARLY0 = CPG > 2;   // chunk 0 of pass 2 before the rest of pass 1
    // numerators of every chunk of the group (registers), normalisers in LDS
    f32x4 O[CPG][4];
    // the state before the group: wait for the earlier groups' flags, sum
    // their published states (each wave its columns' Z tiles and its S
    // tiles), correct chunk 0 (numerators += column sums of Ze + Ze^T psi(q),
    // own normaliser += sum Se + Se . psi(q)), then add it to the running
    // state and to the next chunk's S operands
    auto look_back = [&]() __attribute__((always_inline)) {
        __syncthreads();   // every wave is done with chunk 0's S operands (buffer 0)
        load_state(Ze, Se, nullptr, nullptr);
        bool ok;
        const bool local = wait_flags(a.flags + (int64_t)hp * a.G, 1, grp, a.wait_tag, my_xcc, lane, a.spin_limit, ok);
        constexpr int LB = JT <= 4 ? 4 : 2;   // slots in flight (register budget)
        const char *base = (const char *)a.part + (size_t)hp * a.G * FS::BYTES;
        auto sum = [&](auto cpol) __attribute__((always_inline)) {
            constexpr int CP = decltype(cpol)::value;
            for (int g0 = 0; g0 < grp; g0 += LB) {
                f32x4 tz[LB][JT], ts[LB][SPW];
#pragma unroll
                for (int u = 0; u < LB; ++u) {
                    const bool live = g0 + u < grp;
                    const rsrc_t sr = make_rsrc(base + (size_t)(live ? g0 + u : 0) * FS::BYTES, live ? FS::BYTES : 0);
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) tz[u][jt] = dload16<CP>(sr, FS::zoff(w, jt, lane));
#pragma unroll
                    for (int m = 0; m < SPW; ++m) ts[u][m] = dload16<CP>(sr, FS::soff(w + NWAVE * m, g));
                }
#pragma unroll
                for (int u = 0; u < LB; ++u) {
#pragma unroll
                    for (int jt = 0; jt < JT; ++jt) Ze[jt] += tz[u][jt];
#pragma unroll
                    for (int m = 0; m < SPW; ++m) Se[m] += ts[u][m];
                }
            }
        };
        if (local) sum(IC<CPOL_XCD>{});
        else sum(IC<CPOL_DEVICE>{});
        if (!ok) {   // the earlier groups' state is unknown: poison it
            count_giveup(a.giveups, lane);
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) Ze[jt] = (f32x4){NAN, NAN, NAN, NAN};
#pragma unroll
            for (int m = 0; m < SPW; ++m) Se[m] = (f32x4){NAN, NAN, NAN, NAN};
        }
        put_sops(Se, 0);
        __syncthreads();
        bf16x8 zh[KS], zl[KS];
        f32x4 cz;
        state_ops(Ze, zh, zl, cz);
        const bf16 *Qb = qslot(0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            bf16x8 qb[KS];
            q_ops(Qb, m, qb);
            f32x4 o = O[0][m] + cz;
#pragma unroll
            for (int u = 0; u < KS; ++u) {
                o = mma8(o, zh[u], qb[u]);
                o = mma8(o, zl[u], qb[u]);
            }
            O[0][m] = o;
            if (m == w) {
                const f32x4 dn = sdot(0, qb);
                if (g == 0) den_s[16 * m + r] += dn[0];
            }
        }
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) Z[jt] += Ze[jt];
#pragma unroll
        for (int m = 0; m < SPW; ++m) S[m] += Se[m];
        if (nch > 1) put_sops(S, 1);
    };
    // the outputs of chunk c: numerators / normalisers (every normaliser of
    // the chunk is complete after the next barrier)
    auto store_out = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        const int t0 = t_begin + c * C, nv = nval_of(c);
        const rsrc_t orr = ov.at(t0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int t = 16 * m + r;
            const float inv = UNNORM ? 1.f : __builtin_amdgcn_rcpf(den_s[c * C + t] + a.eps);
            bstore16nt(orr, t < nv ? (uint32_t)(t * ov.rs + (16 * w + 4 * g) * 4) : OFF_NONE, O[c][m] * inv);
        }
    };
    // one chunk of pass 2, everything but the next chunk's stage.  Per
    // chunk: barrier; scores, inter term, state update (every read of this
    // chunk's psi(K) and V); barrier; P V, normaliser.
    auto chunk = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        const int buf = c & 1, nv = nval_of(c);
        __syncthreads();   // the stage is visible; the previous chunk's second half is done
        __builtin_amdgcn_s_setprio(CPG - 1 - c);   // progress-based priority (see pass 1)
        if constexpr (!EARLY0 && c + 2 < CPG) issue_q(IC<c + 2>{});
        const bf16 *Kb = kbuf(), *Qb = qslot(c), *Vb = vbuf();
        // this wave's score tiles: three table entries (sa, m) per wave,
        // 4 bits each; waves 2 and 3 repeat tile (0, 0), which writes the
        // same values as wave 0
        //   w0: (0,0) (0,3) (1,3)   w1: (0,1) (1,1) (2,3)
        //   w2: (0,2) (1,2) (0,0)   w3: (2,2) (3,3) (0,0)
        {
            const uint32_t tab = (0x000000u | 0x03u << 8 | 0x13u << 16) * (w == 0) +
                                 (0x01u | 0x11u << 8 | 0x23u << 16) * (w == 1) +
                                 (0x02u | 0x12u << 8 | 0x00u << 16) * (w == 2) +
                                 (0x22u | 0x33u << 8 | 0x00u << 16) * (w == 3);
            constexpr int TR = KS <= 2 ? 3 : 1;   // tiles whose operands are read together
#pragma unroll
            for (int i0 = 0; i0 < 3; i0 += TR) {
                bf16x8 ka[TR][KS], qa[TR][KS];
#pragma unroll
                for (int i = 0; i < TR; ++i) {
                    const int e = (tab >> (8 * (i0 + i))) & 0xff;
#pragma unroll
                    for (int u = 0; u < KS; ++u) {
                        ka[i][u] = nat8(Kb + swz<D>(16 * (e >> 4) + r, 32 * u + 8 * g));
                        qa[i][u] = nat8(Qb + swz<D>(16 * (e & 15) + r, 32 * u + 8 * g));
                    }
                }
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int i = 0; i < TR; ++i) {
                    const int e = (tab >> (8 * (i0 + i))) & 0xff;
                    score_tile(ka[i], qa[i], e >> 4, e & 15, nv, buf, c);
                }
            }
        }
        if constexpr (c > 0) store_out(IC<c - 1>{});   // the previous chunk is complete
        // inter-chunk term of every query tile: column sums of Z plus
        // Z^T psi(q)
        f32x4 o[4];
        {
            bf16x8 zh[KS], zl[KS];
            f32x4 cz;
            state_ops(Z, zh, zl, cz);
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                bf16x8 qb[KS];
                q_ops(Qb, m, qb);
                o[m] = cz;
#pragma unroll
                for (int u = 0; u < KS; ++u) {
                    o[m] = mma8(o[m], zh[u], qb[u]);
                    o[m] = mma8(o[m], zl[u], qb[u]);
                }
            }
        }
        // state update (V stays in registers for P V), and this wave's
        // share of the S operands of the next chunk
        bf16x8 va[2];
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) va[sg] = tr8<64>(Vb, 32 * sg, 16 * w, r, g);
        update_state(Kb, va, nv);
        if (c + 1 < nch) put_sops(S, buf ^ 1);
        __syncthreads();   // the score operands are visible; this chunk's psi(K) and V are read
        // intra-chunk term: V^T P^T over key tile pairs (2sg, 2sg + 1)
        {
            bf16x8 pp[6][2];   // the 6 score operand pairs, read before the products
#pragma unroll
            for (int pr = 0; pr < 6; ++pr) { pp[pr][0] = nat8(pop_at(pr, 0, lane)); pp[pr][1] = nat8(pop_at(pr, 1, lane)); }
#pragma unroll
            for (int m = 0; m < 4; ++m) {
#pragma unroll
                for (int sg = 0; 2 * sg <= m; ++sg) {
                    o[m] = mma8(o[m], va[sg], pp[pbase(m) + sg][0]);
                    o[m] = mma8(o[m], va[sg], pp[pbase(m) + sg][1]);
                }
                O[c][m] = o[m];
            }
        }
        // normaliser of this wave's query tile w: sum_i S_i + S . psi(q) +
        // sum_s P (the second key pair only for w >= 2: a zero operand
        // otherwise)
        {
            bf16x8 qw[KS];
            q_ops(Qb, w, qw);
            f32x4 dn = sdot(buf, qw), dp = {0.f, 0.f, 0.f, 0.f};   // two independent chains
            const int pw = pbase(w);
            const bf16x8 z8 = {};
            const bool two = w >= 2;
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                bf16x8 ph = nat8(pop_at(pw + (sg & (int)two), 0, lane)), pl = nat8(pop_at(pw + (sg & (int)two), 1, lane));
                if (sg == 1) { ph = two ? ph : z8; pl = two ? pl : z8; }
                dp = mma8(dp, ones8, ph);
                dp = mma8(dp, ones8, pl);
            }
            dn += dp;
            if (g == 0) den_s[c * C + 16 * w + r] = dn[0];
        }
    };
    // pass 1 for chunk c: k turned into psi(k) in its registers; every
    // group but the last adds psi(K)^T V to its running state
    auto pass1_chunk = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value;
        stage_kv(cc);
        if constexpr (EARLY0) {   // loads run two chunks ahead of their use
            if constexpr (c + 2 < CPG) issue_kv(IC<c + 2>{});
            issue_q(cc);
        } else if constexpr (c == 0) {   // q of the first two chunks is requested meanwhile
            issue_q(IC<0>{});
            if constexpr (CPG > 1) issue_q(IC<1>{});
        }
        if (!last) {
            __syncthreads();   // the stage is visible
            bf16x8 va[2];
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) va[sg] = tr8<64>(vbuf(), 32 * sg, 16 * w, r, g);
            update_state(kbuf(), va, nval_of(c));
            __syncthreads();   // the stage is read
        }
    };
    // the group's partial state to its slot, then the flag: this
    // workgroup's memory accesses (slot stores; group 0: its reads of the
    // carried-in state) are complete.  A last group 0 sets it only to signal
    // that s_in has been read.
    auto publish = [&]() __attribute__((always_inline)) {
        if (!last) {
            const rsrc_t sr = make_rsrc((const char *)a.part + (size_t)(hp * a.G + grp) * FS::BYTES, FS::BYTES);
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) dstore16(sr, FS::zoff(w, jt, lane), Z[jt]);
#pragma unroll
            for (int m = 0; m < SPW; ++m) dstore16(sr, r == 0 ? FS::soff(w + NWAVE * m, g) : OFF_NONE, S[m]);
        }
    };
    auto set_flag = [&]() __attribute__((always_inline)) {
        if (!last || (grp == 0 && a.wait_s)) {
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
            if (tid == 0)
                __hip_atomic_store(a.flags + (int64_t)hp * a.G + grp, a.epoch | my_xcc, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
    };

    // ================= the schedule.  Pass 1 (state only) publishes the
    // group's partial state as early as the loads allow; pass 2 computes the
    // outputs, chunk by chunk against the running state.  At d <= 64 chunk 0
    // of pass 2 runs first, as soon as its inputs arrive (its state is the
    // start state), and the state after it is kept while pass 1 advances
    // over the remaining chunks.  At d = 128 (two chunks per group, so pass 1
    // is short and publishing early matters more) pass 1 covers every chunk
    // first and the start state is loaded again.  Then the state
    // before the group is looked up (groups after the first) and chunk 0
    // corrected, so chunks 1.. see the full prefix.
    // Wave priorities follow progress: the two workgroups that share a CU
    // would otherwise run oldest-first, and the younger one would finish its
    // last chunks alone on the CU.  Pass 1 and chunk 0 run at the top
    // priority, chunk c of pass 2 at CPG - 1 - c, so a workgroup that is
    // ahead yields.
    static_assert(CPG >= 1 && CPG <= 4, "priorities 0..3 cover the chunks");
    __builtin_amdgcn_s_setprio(3);
    if constexpr (EARLY0) {
        // the loads are requested in the order of use, at most two chunks
        // ahead, so that the first chunks of every workgroup arrive first
        load_start();
        issue_kv(IC<0>{});
        issue_q(IC<0>{});
        put_sops(S, 0);
        stage_kv(IC<0>{});   // psi(k) of chunk 0 (its state update is part of chunk 0 below)
        stage(IC<0>{});
        if constexpr (CPG > 1) issue_kv(IC<1>{});
        if constexpr (CPG > 2) issue_kv(IC<2>{});
        if (nch > 0) chunk(IC<0>{});   // always; keeps chunk 0 a region of its own for the scheduler
        __builtin_amdgcn_s_setprio(3);
        f32x4 Zs[JT], Ss[SPW];   // the state after chunk 0
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) Zs[jt] = Z[jt];
#pragma unroll
        for (int m = 0; m < SPW; ++m) Ss[m] = S[m];
        static_for<CPG>([&](auto cc) {
            if constexpr (cc.value > 0)
                if (cc.value < nch) pass1_chunk(cc);
        });
        publish();
        set_flag();
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) Z[jt] = Zs[jt];
#pragma unroll
        for (int m = 0; m < SPW; ++m) S[m] = Ss[m];
        if constexpr (CPG > 1) stage(IC<1>{});
        if (grp > 0) look_back();
    } else {
        if (!last) load_start();
        static_for<CPG>([&](auto cc) { issue_kv(cc); });
        static_for<CPG>([&](auto cc) {
            constexpr int c = decltype(cc)::value;
            if (c < nch) pass1_chunk(cc);
        });
        publish();
        // the start state of pass 2, read again (group 0) before the flag, so
        // that a last group writing the final state in place never overtakes it
        load_start();
        set_flag();
        put_sops(S, 0);
        stage(IC<0>{});
        if (nch > 0) {   // always; keeps chunk 0 a region of its own for the scheduler
            chunk(IC<0>{});
            if constexpr (CPG > 1) stage(IC<1>{});
            if (grp > 0) look_back();
        }
    }
    static_for<CPG>([&](auto cc) {
        constexpr int c = decltype(cc)::value;
        if constexpr (c > 0) {
            if (c < nch) {
                chunk(cc);
                // the next chunk's stage (chunks past the group stage zeros,
                // never read); its VALU work can be scheduled between the
                // products above
                if constexpr (c + 1 < CPG) stage(IC<c + 1>{});
            }
        }
    });
    __syncthreads();   // the last chunk's normalisers are complete
    static_for<CPG>([&](auto cc) {
        if (cc.value == nch - 1) store_out(cc);
    });
    // ---- the final state (last group): the running state after the last chunk
    if (last) {
        if (a.wait_s && s_writer) {
            bool ok;
            (void)wait_flags(a.flags + (int64_t)bh * a.P * a.G, a.G, a.P, a.wait_tag, my_xcc, lane, a.spin_limit, ok);
            if (!ok) {   // s_in may not have been read yet: poison s_out
                count_giveup(a.giveups, lane);
#pragma unroll
                for (int m = 0; m < SPW; ++m) S[m] = (f32x4){NAN, NAN, NAN, NAN};
            }
        }
        float *zo = a.z_out ? a.z_out + (int64_t)bh * D * D + p * DV + 16 * w + r : nullptr;
        float *so = (a.s_out && s_writer && r == 0) ? a.s_out + (int64_t)bh * D : nullptr;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (zo) zo[(int64_t)cs_dim(jt, 4 * g + i) * D] = Z[jt][i];
            }
#pragma unroll
        for (int m = 0; m < SPW; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (so) so[cs_dim(w + NWAVE * m, 4 * g + i)] = S[m][i];
            }
    }
}

// ================================================================ non-causal, column split
// (bf16 inputs, 64-token chunks, DV = 64 columns per workgroup, each wave 16)
//
// k_cs_state: the partial state of one share of the tokens, Z[:, block] =
// sum_t phi(k_t) v_t^T and S = sum_t phi(k_t), written to slot grp of
// (head, column block) in the layout of the state tensors ([D][DV] row major,
// then S [D]).  phi = 1 + psi: Z += psi(K)^T V + 1 (column sums of V)^T,
// S += psi(K)^T 1 + tokens, with psi(K) in bf16 and V as loaded.  Share grp
// of G takes the 64-token chunks grp, grp + G, grp + 2G, ... (the G
// workgroups of a head read neighbouring chunks at any one time).
template <int D>
__global__ void __launch_bounds__(NTHR, D <= 64 ? 4 : 2) k_cs_state(const Args a)
{
    typedef CSGeo<D> T;
    constexpr int C = T::C, DV = T::DV, JT = T::JT, VPR = T::VPR, NK = T::NK, NV = T::NV;
    constexpr int SL = Slot<D, DV>::SIZE;
    __shared__ __attribute__((aligned(16))) bf16 sm[2 * C * D + 2 * C * DV];   // psi(K) [2][C][D], V [2][C][DV]
    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int p = wg % a.P, rest = wg / a.P, grp = rest % a.G, bh = rest / a.G;
    const int b = bh / a.H, h = bh % a.H;
    const int hp = bh * a.P + p;
    const int nall = (a.N + C - 1) / C;                    // chunks of the sequence
    const int nch = grp < nall ? (nall - grp + a.G - 1) / a.G : 0;   // chunks of this share
    auto t0_of = [&](int ch) { return (grp + ch * a.G) * C; };
    const RowView kv{(const char *)a.k + (b * a.skb + h * a.skh) * 2, a.skn * 2, (a.N - 1) * a.skn * 2 + D * 2};
    const RowView vv{(const char *)a.v + (b * a.svb + h * a.svh + p * DV) * 2, a.svn * 2,
                     (a.N - 1) * a.svn * 2 + DV * 2};
    uint32_t ko[NK], vo[NV];
#pragma unroll
    for (int it = 0; it < NK; ++it) {
        const int item = tid + it * NTHR;
        ko[it] = (uint32_t)((item / VPR) * kv.rs + (item % VPR) * 16);
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
        const int item = tid + it * NTHR;
        vo[it] = (uint32_t)((item / 8) * vv.rs + (item % 8) * 16);
    }
    u32x4 Kr[2][NK], Vr[2][NV];   // chunks ch + 1 and ch + 2 in flight
    auto issue = [&](int ch, int slot) {
        const int t0 = ch < nch ? t0_of(ch) : 0;
        const rsrc_t kr = kv.at(t0, ch < nch), vr = vv.at(t0, ch < nch);
#pragma unroll
        for (int it = 0; it < NK; ++it) Kr[slot][it] = bload16nt(kr, ko[it]);
#pragma unroll
        for (int it = 0; it < NV; ++it) Vr[slot][it] = bload16nt(vr, vo[it]);
    };
    bf16x8 ones8;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones8[e] = (bf16)1.f;
    f32x4 Z[JT], S[JT];
#pragma unroll
    for (int jt = 0; jt < JT; ++jt) { Z[jt] = (f32x4){0.f, 0.f, 0.f, 0.f}; S[jt] = Z[jt]; }
    float ntok = 0.f;
    // one chunk from register slot `slot` through stage buffer `buf`
    auto step = [&](int ch, int slot, int buf) {
        bf16 *Kb = sm + buf * C * D, *Vb = sm + 2 * C * D + buf * C * DV;
#pragma unroll
        for (int it = 0; it < NK; ++it) {
            const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
            *reinterpret_cast<u32x4 *>(Kb + swz<D>(row, vec * 8)) = cs_psi8(Kr[slot][it]);
        }
#pragma unroll
        for (int it = 0; it < NV; ++it) {
            const int item = tid + it * NTHR, row = item / 8, vec = item % 8;
            *reinterpret_cast<u32x4 *>(Vb + swz<64>(row, vec * 8)) = Vr[slot][it];
        }
        issue(ch + 2, slot);
        __syncthreads();   // the stage is visible; the other buffer's readers are done
        bf16x8 va[2];
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) va[sg] = tr8<64>(Vb, 32 * sg, 16 * w, r, g);
        bf16x8 kt[JT][2];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) kt[jt][sg] = cs_ktr8<D>(Kb, 32 * sg, jt, r, g);
        f32x4 cv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int sg = 0; sg < 2; ++sg) cv = mma8(cv, ones8, va[sg]);
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) {
                Z[jt] = mma8(Z[jt], kt[jt][sg], va[sg]);
                S[jt] = mma8(S[jt], kt[jt][sg], ones8);
            }
            Z[jt] += cv;
        }
        ntok += ch < nch ? (float)min(C, a.N - t0_of(ch)) : 0.f;   // 0 for the empty step
    };
    issue(0, 0);
    issue(1, 1);
    for (int ch = 0; ch < nch; ch += 2) {   // an odd count runs one empty step (zeros)
        step(ch, 0, 0);
        step(ch + 1, 1, 1);
    }
    if (a.direct) {
        // one share per (head, column block): the final state itself,
        // z_out = z_in + Z and (column block 0) s_out = s_in + S; each
        // element is read and written by one thread, so in place is safe
        const int64_t zo = (int64_t)bh * D * D + p * DV + 16 * w + r;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dim = cs_dim(jt, 4 * g + i);
                if (a.z_out) a.z_out[zo + dim * D] = Z[jt][i] + (a.z_in ? a.z_in[zo + dim * D] : 0.f);
                if (a.s_out && p == 0 && w == 0 && r == 0)
                    a.s_out[(int64_t)bh * D + dim] = S[jt][i] + ntok + (a.s_in ? a.s_in[(int64_t)bh * D + dim] : 0.f);
            }
        return;
    }
    // the slot: Z in [D][DV] layout, S (wave 0)
    float *slot = a.part + ((int64_t)hp * a.NS + grp) * SL;
#pragma unroll
    for (int jt = 0; jt < JT; ++jt)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int dim = cs_dim(jt, 4 * g + i);
            slot[dim * DV + 16 * w + r] = Z[jt][i];
            if (w == 0 && r == 0) slot[DV * D + dim] = S[jt][i] + ntok;
        }
}

// k_cs_apply: out_t = phi(q_t)^T Z / (phi(q_t) . S + eps) for a group of
// tokens against the reduced global state (fin [hp] in the slot layout):
// numerator = sum_i Z[i][:] + Z^T psi(q_t), normaliser = sum_i S_i +
// S . psi(q_t), with Z and S as bf16 hi + lo operands.  Every wave computes
// the normalisers of all queries (no exchange).
template <int D>
__global__ void __launch_bounds__(NTHR, D <= 64 ? 4 : 2) k_cs_apply(const Args a)
{
    typedef CSGeo<D> T;
    constexpr int C = T::C, DV = T::DV, JT = T::JT, KS = T::KS, VPR = T::VPR, NK = T::NK;
    constexpr int SL = Slot<D, DV>::SIZE;
    __shared__ __attribute__((aligned(16))) bf16 sm[2 * C * D];   // psi(Q) [2][C][D]
    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int wg = xcd_remap(blockIdx.x, gridDim.x);
    const int p = wg % a.P, rest = wg / a.P, grp = rest % a.G, bh = rest / a.G;
    const int b = bh / a.H, h = bh % a.H;
    const int hp = bh * a.P + p;
    const int t_begin = grp * a.L, t_end = min(t_begin + a.L, a.N);
    const int nch = (t_end - t_begin + C - 1) / C;
    const RowView qv{(const char *)a.q + (b * a.sqb + h * a.sqh) * 2, a.sqn * 2, (a.N - 1) * a.sqn * 2 + D * 2};
    const RowView ov{(const char *)(a.out + b * a.sob + h * a.soh + p * DV), a.son * 4, (a.N - 1) * a.son * 4 + DV * 4};
    uint32_t qo[NK];
#pragma unroll
    for (int it = 0; it < NK; ++it) {
        const int item = tid + it * NTHR;
        qo[it] = (uint32_t)((item / VPR) * qv.rs + (item % VPR) * 16);
    }
    u32x4 Qr[2][NK];
    auto issue = [&](int ch, int slot) {
        const rsrc_t qr = qv.at(t_begin + ch * C, ch < nch);
#pragma unroll
        for (int it = 0; it < NK; ++it) Qr[slot][it] = bload16nt(qr, qo[it]);
    };
    issue(0, 0);
    issue(1, 1);
    bf16x8 ones8;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones8[e] = (bf16)1.f;
    // the state's operands: Z (this wave's 16 columns) and S, hi + lo, and
    // their sums over the key dims
    const float *fin = a.fin + (int64_t)hp * SL;
    bf16x8 zh[KS], zl[KS], sh[KS], sl[KS];
    f32x4 cz = {0.f, 0.f, 0.f, 0.f}, cs = cz;
    {
        f32x4 Z[JT], S[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dim = cs_dim(jt, 4 * g + i);
                Z[jt][i] = fin[dim * DV + 16 * w + r];
                S[jt][i] = fin[DV * D + dim];
            }
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            cs_split(Z[2 * u], Z[2 * u + 1], zh[u], zl[u]);
            cs_split(S[2 * u], S[2 * u + 1], sh[u], sl[u]);
            cz = mma8(cz, zh[u], ones8);
            cz = mma8(cz, zl[u], ones8);
            cs = mma8(cs, sh[u], ones8);
            cs = mma8(cs, sl[u], ones8);
        }
    }
    auto step = [&](int ch, int slot, int buf) {
        bf16 *Qb = sm + buf * C * D;
#pragma unroll
        for (int it = 0; it < NK; ++it) {
            const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
            *reinterpret_cast<u32x4 *>(Qb + swz<D>(row, vec * 8)) = cs_psi8(Qr[slot][it]);
        }
        issue(ch + 2, slot);
        __syncthreads();   // the stage is visible; the other buffer's readers are done
        const int t0 = t_begin + ch * C, nv = min(C, t_end - t0);
        const rsrc_t orr = ov.at(t0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            bf16x8 qb[KS];
#pragma unroll
            for (int u = 0; u < KS; ++u) qb[u] = nat8(Qb + swz<D>(16 * m + r, 32 * u + 8 * g));
            f32x4 o = cz, dn = cs;
#pragma unroll
            for (int u = 0; u < KS; ++u) {
                o = mma8(o, zh[u], qb[u]);
                o = mma8(o, zl[u], qb[u]);
                dn = mma8(dn, sh[u], qb[u]);
                dn = mma8(dn, sl[u], qb[u]);
            }
            // dn holds the normaliser of query r in every row
            const float inv = __builtin_amdgcn_rcpf(dn[0] + a.eps);
            const int t = 16 * m + r;
            bstore16(orr, t < nv ? (uint32_t)(t * ov.rs + (16 * w + 4 * g) * 4) : OFF_NONE, o * inv);
        }
    };
    for (int ch = 0; ch < nch; ch += 2) {
        step(ch, 0, 0);
        if (ch + 1 < nch) step(ch + 1, 1, 1);
    }
}

// k_cs_memory: a compressive-memory call in one launch of two workgroups per
// token share (share grp of G takes the 64-token chunks grp, grp + G, ...).
// The reads of the memory need only the carried-in state, not the segment's,
// so the two jobs run side by side: an even workgroup forms the share's
// partial state, Z = sum psi(k) v^T + 1 (sum v)^T and S = sum psi(k) + tokens
// (as k_cs_state; each wave forms only its S tiles w, w + 4, ...), and writes
// it to the share's slot; the odd one lets every query of the share read the
// carried-in memory, out_t = phi(q_t)^T Z_in / (phi(q_t) . S_in + eps) (as
// k_cs_apply, with Z_in and S_in read from the state tensors).  k_slots then
// adds the slots to the memory.
template <int D>
__global__ void __launch_bounds__(NTHR, 2) k_cs_memory(const Args a)
{
    typedef CSGeo<D> T;
    constexpr int C = T::C, DV = T::DV, JT = T::JT, KS = T::KS, VPR = T::VPR, NK = T::NK, NV = T::NV;
    constexpr int SL = Slot<D, DV>::SIZE;
    constexpr int SPW = JT / NWAVE;
    static_assert(JT % NWAVE == 0, "S tiles split evenly over the waves");
    // state: psi(K) [2][C][D], V [2][C][DV]; reads: psi(Q) [2][C][D]
    __shared__ __attribute__((aligned(16))) bf16 sm[2 * C * D + 2 * C * DV];
    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int wg2 = xcd_remap(blockIdx.x, gridDim.x);
    const bool reader = wg2 & 1;   // odd workgroups read the memory, even ones form the partial states
    const int wg = wg2 >> 1;
    const int p = wg % a.P, rest = wg / a.P, grp = rest % a.G, bh = rest / a.G;
    const int b = bh / a.H, h = bh % a.H;
    const int hp = bh * a.P + p;
    const int nall = (a.N + C - 1) / C;
    const int nch = grp < nall ? (nall - grp + a.G - 1) / a.G : 0;
    auto t0_of = [&](int ch) { return (grp + ch * a.G) * C; };
    const RowView qv{(const char *)a.q + (b * a.sqb + h * a.sqh) * 2, a.sqn * 2, (a.N - 1) * a.sqn * 2 + D * 2};
    const RowView kv{(const char *)a.k + (b * a.skb + h * a.skh) * 2, a.skn * 2, (a.N - 1) * a.skn * 2 + D * 2};
    const RowView vv{(const char *)a.v + (b * a.svb + h * a.svh + p * DV) * 2, a.svn * 2,
                     (a.N - 1) * a.svn * 2 + DV * 2};
    const RowView ov{(const char *)(a.out + b * a.sob + h * a.soh + p * DV), a.son * 4, (a.N - 1) * a.son * 4 + DV * 4};
    uint32_t qo[NK], ko[NK], vo[NV];
#pragma unroll
    for (int it = 0; it < NK; ++it) {
        const int item = tid + it * NTHR;
        qo[it] = (uint32_t)((item / VPR) * qv.rs + (item % VPR) * 16);
        ko[it] = (uint32_t)((item / VPR) * kv.rs + (item % VPR) * 16);
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
        const int item = tid + it * NTHR;
        vo[it] = (uint32_t)((item / 8) * vv.rs + (item % 8) * 16);
    }
    bf16x8 ones8;
#pragma unroll
    for (int e = 0; e < 8; ++e) ones8[e] = (bf16)1.f;
    u32x4 Qr[2][NK];   // q of chunks ch + 1 and ch + 2 in flight (reads)
    auto issue_q = [&](int ch, int slot) {
        const rsrc_t qr = qv.at(ch < nch ? t0_of(ch) : 0, ch < nch);
#pragma unroll
        for (int it = 0; it < NK; ++it) Qr[slot][it] = bload16nt(qr, qo[it]);
    };

    // ================= even workgroups: the share's partial state
    if (!reader) {
        u32x4 Kr[2][NK], Vr[2][NV];   // chunks ch + 1 and ch + 2 in flight
        auto issue_kv = [&](int ch, int slot) {
            const int t0 = ch < nch ? t0_of(ch) : 0;
            const rsrc_t kr = kv.at(t0, ch < nch), vr = vv.at(t0, ch < nch);
#pragma unroll
            for (int it = 0; it < NK; ++it) Kr[slot][it] = bload16nt(kr, ko[it]);
#pragma unroll
            for (int it = 0; it < NV; ++it) Vr[slot][it] = bload16nt(vr, vo[it]);
        };
        issue_kv(0, 0);
        issue_kv(1, 1);
        f32x4 Z[JT], S[SPW];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) Z[jt] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < SPW; ++m) S[m] = (f32x4){0.f, 0.f, 0.f, 0.f};
        float ntok = 0.f;
        auto step = [&](int ch, int slot, int buf) {
            bf16 *Kb = sm + buf * C * D, *Vb = sm + 2 * C * D + buf * C * DV;
#pragma unroll
            for (int it = 0; it < NK; ++it) {
                const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
                *reinterpret_cast<u32x4 *>(Kb + swz<D>(row, vec * 8)) = cs_psi8(Kr[slot][it]);
            }
#pragma unroll
            for (int it = 0; it < NV; ++it) {
                const int item = tid + it * NTHR, row = item / 8, vec = item % 8;
                *reinterpret_cast<u32x4 *>(Vb + swz<64>(row, vec * 8)) = Vr[slot][it];
            }
            issue_kv(ch + 2, slot);
            __syncthreads();   // the stage is visible; the other buffer's readers are done
            bf16x8 va[2];
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) va[sg] = tr8<64>(Vb, 32 * sg, 16 * w, r, g);
            f32x4 cv = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int sg = 0; sg < 2; ++sg) cv = mma8(cv, ones8, va[sg]);
            constexpr int JR = 2;   // state tiles whose operands are read together
#pragma unroll
            for (int j0 = 0; j0 < JT; j0 += JR) {
                bf16x8 kt[JR][2];
#pragma unroll
                for (int j = 0; j < JR; ++j)
#pragma unroll
                    for (int sg = 0; sg < 2; ++sg) kt[j][sg] = cs_ktr8<D>(Kb, 32 * sg, j0 + j, r, g);
#pragma unroll
                for (int j = 0; j < JR; ++j) {
#pragma unroll
                    for (int sg = 0; sg < 2; ++sg) Z[j0 + j] = mma8(Z[j0 + j], kt[j][sg], va[sg]);
                    Z[j0 + j] += cv;
                }
            }
#pragma unroll
            for (int m = 0; m < SPW; ++m)
#pragma unroll
                for (int sg = 0; sg < 2; ++sg) S[m] = mma8(S[m], cs_ktr8<D>(Kb, 32 * sg, w + NWAVE * m, r, g), ones8);
            ntok += ch < nch ? (float)min(C, a.N - t0_of(ch)) : 0.f;   // 0 for the empty step
        };
        for (int ch = 0; ch < nch; ch += 2) {   // an odd count runs one empty step (zeros)
            step(ch, 0, 0);
            step(ch + 1, 1, 1);
        }
        float *slot = a.part + ((int64_t)hp * a.NS + grp) * SL;
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) slot[cs_dim(jt, 4 * g + i) * DV + 16 * w + r] = Z[jt][i];
#pragma unroll
        for (int m = 0; m < SPW; ++m)
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (r == 0) slot[DV * D + cs_dim(w + NWAVE * m, 4 * g + i)] = S[m][i] + ntok;
        return;
    }

    // ================= odd workgroups: every query reads the carried-in memory
    issue_q(0, 0);
    issue_q(1, 1);
    bf16x8 zh[KS], zl[KS], sh[KS], sl[KS];
    f32x4 cz = {0.f, 0.f, 0.f, 0.f}, cs = cz;
    {
        const float *zin = a.z_in ? a.z_in + (int64_t)bh * D * D + p * DV + 16 * w + r : nullptr;
        const float *sin = a.s_in ? a.s_in + (int64_t)bh * D : nullptr;
        f32x4 Zm[JT], Sm[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int dim = cs_dim(jt, 4 * g + i);
                Zm[jt][i] = zin ? zin[(int64_t)dim * D] : 0.f;
                Sm[jt][i] = sin ? sin[dim] : 0.f;
            }
#pragma unroll
        for (int u = 0; u < KS; ++u) {
            cs_split(Zm[2 * u], Zm[2 * u + 1], zh[u], zl[u]);
            cs_split(Sm[2 * u], Sm[2 * u + 1], sh[u], sl[u]);
            cz = mma8(cz, zh[u], ones8);
            cz = mma8(cz, zl[u], ones8);
            cs = mma8(cs, sh[u], ones8);
            cs = mma8(cs, sl[u], ones8);
        }
    }
    auto read = [&](int ch, int slot, int buf) {
        bf16 *Qb = sm + buf * C * D;
#pragma unroll
        for (int it = 0; it < NK; ++it) {
            const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
            *reinterpret_cast<u32x4 *>(Qb + swz<D>(row, vec * 8)) = cs_psi8(Qr[slot][it]);
        }
        issue_q(ch + 2, slot);
        __syncthreads();   // the stage is visible; the other buffer's readers are done
        const int t0 = ch < nch ? t0_of(ch) : 0, nv = ch < nch ? min(C, a.N - t0) : 0;
        const rsrc_t orr = ov.at(t0, nv > 0);
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            bf16x8 qb[KS];
#pragma unroll
            for (int u = 0; u < KS; ++u) qb[u] = nat8(Qb + swz<D>(16 * m + r, 32 * u + 8 * g));
            f32x4 o = cz, dn = cs;
#pragma unroll
            for (int u = 0; u < KS; ++u) {
                o = mma8(o, zh[u], qb[u]);
                o = mma8(o, zl[u], qb[u]);
                dn = mma8(dn, sh[u], qb[u]);
                dn = mma8(dn, sl[u], qb[u]);
            }
            // dn holds the normaliser of query r in every row
            const float inv = __builtin_amdgcn_rcpf(dn[0] + a.eps);
            const int t = 16 * m + r;
            bstore16nt(orr, t < nv ? (uint32_t)(t * ov.rs + (16 * w + 4 * g) * 4) : OFF_NONE, o * inv);
        }
    };
    for (int ch = 0; ch < nch; ch += 2) {
        read(ch, 0, 0);
        if (ch + 1 < nch) read(ch + 1, 1, 1);
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
    // the state rows are requested first (they do not depend on phi), with
    // non-temporal hints: each element is read and written once per step
    float *zh = z + (int64_t)(active ? bh : 0) * D * D + 4 * cq;
    f32x4 zr[RPT];
    if (active) {
#pragma unroll
        for (int m = 0; m < RPT; ++m)
            zr[m] = __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(zh + (int64_t)(m * RG + rg) * D));
    }
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
#pragma unroll
        for (int m = 0; m < RPT; ++m) {
            const int j = m * RG + rg;
            const float fj = sphik[hl][j];
            zr[m] += fj * vv;
            __builtin_nontemporal_store(zr[m], reinterpret_cast<f32x4 *>(zh + (int64_t)j * D));
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

// ================================================================ backward pass
// Gradients of the causal form (the backward pass of training, which
// "Attention Kernel Mask" lists as a row of its table under "Causal Attention
// Training and Inferencing" without writing it out).  With g_t = phi(q_t),
// f_s = phi(k_s), the running state Z_t, S_t (carried-in state included),
// D_t = g_t . S_t + eps and an upstream gradient dout_t:
//   dn_t = dout_t / D_t,  dD_t = -(dout_t . out_t) / D_t,
//   dq_t = phi'(q_t) * (Z_t dn_t + S_t dD_t),
//   dk_s = phi'(k_s) * (R_s v_s + r_s),  dv_s = R_s^T f_s,
// where R_s = dz_out + sum_{t >= s} g_t dn_t^T and r_s = ds_out + sum_{t >= s}
// g_t dD_t are the adjoint state.  phi'(x) = min(phi(x), 1).
// Per 64-token chunk c (inclusive masks inside the chunk), with A_ts =
// v_s . dn_t + dD_t and P_ts = g_t . f_s:
//   dq_t = phi'(q_t) * (Z_c dn_t + S_c dD_t + sum_{s <= t} A_ts f_s)
//   dk_s = phi'(k_s) * (R'_c v_s + r'_c + sum_{t >= s} A_ts g_t)
//   dv_s = R'_c^T f_s + sum_{t >= s} P_ts dn_t
// where (Z_c, S_c) is the state before the chunk and (R'_c, r'_c) the adjoint
// state after it.  Both are materialised at every chunk boundary (the mode of
// "How to accelerate causal linear attention" that scans all chunk states
// first and then computes every chunk independently): the forward states by
// k_group_state + a k_slots scan, the adjoint ones by k_bwd_prep + a k_slots
// scan over reverse-indexed slots.  Every product runs on fp32 MFMA.
struct BwdArgs {
    const void *q, *k, *v;
    const float *out, *dout;
    int64_t sqb, sqh, sqn, skb, skh, skn, svb, svh, svn, sob, soh, son, sdb, sdh, sdn;
    float *dq, *dk, *dv;
    int64_t gqb, gqh, gqn, gkb, gkh, gkn, gvb, gvh, gvn;
    int B, H, N, nch, P, NS;
    float eps;
    const float *fwd;   // forward slots [B*H*P][NS]: slot c = the state before chunk c
    float *rev;         // adjoint slots: chunk c writes slot nch - c; after the scan slot nch - 1 - c is
                        // the adjoint state after chunk c
    float *den, *dden;  // D_t and dD_t [B*H][N]
};

// Stage 64 rows (a chunk) of one head into an fp32 [64][D + 4] LDS array.
// MODE 0: the values; 1: phi of the values, zero from row `nval` on; 2: the
// values times 1 / den[row] (zero from row `nval` on).
template <bool F32, int D, int MODE>
__device__ __forceinline__ void bwd_stage(rsrc_t src, int64_t rs, float *dst, int nval, int tid,
                                          const float *den = nullptr)
{
    constexpr int VEC = F32 ? 4 : 8, VPR = D / VEC, ITEMS = 64 * VPR, LD = D + 4;
    static_assert(ITEMS % NTHR == 0, "whole 16-byte vectors per thread");
    u32x4 raw[ITEMS / NTHR];
#pragma unroll
    for (int it = 0; it < ITEMS / NTHR; ++it) {
        const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
        raw[it] = bload16(src, (uint32_t)(row * rs + vec * 16));
    }
#pragma unroll
    for (int it = 0; it < ITEMS / NTHR; ++it) {
        const int item = tid + it * NTHR, row = item / VPR, vec = item % VPR;
        float f[VEC];
        Vec<F32>::to_float(raw[it], f);
        const bool live = row < nval;
        const float scale = MODE == 2 ? (live ? 1.f / den[row] : 0.f) : 1.f;
#pragma unroll
        for (int e = 0; e < VEC; ++e) {
            if (MODE == 1) f[e] = live ? phi<F32>(f[e]) : 0.f;
            if (MODE == 2) f[e] *= scale;
        }
        float *p = dst + row * LD + vec * VEC;
#pragma unroll
        for (int e = 0; e < VEC; e += 4) *reinterpret_cast<f32x4 *>(p + e) = (f32x4){f[e], f[e + 1], f[e + 2], f[e + 3]};
    }
}

// The adjoint part of one chunk: D_t and dD_t of its tokens (to den / dden),
// and  dR_c = sum_t g_t dn_t^T,  dr_c = sum_t g_t dD_t  to adjoint slot
// nch - c (every column block holds dr_c).  Wave w owns tokens 16 w .. + 15
// for the normalisers; the state tiles are split over the waves.
template <bool F32, int D>
__global__ void __launch_bounds__(NTHR) k_bwd_prep(const BwdArgs a)
{
    constexpr int C = 64, LD = D + 4, KT = D / 16, DV = D < 64 ? D : 64, SL = DV * D + D, ES = F32 ? 4 : 2;
    __shared__ __attribute__((aligned(16))) float sm[3 * C * LD + C + NTHR];
    float *Gs = sm, *Fs = sm + C * LD, *Ns = sm + 2 * C * LD, *dDs = sm + 3 * C * LD, *red = dDs + C;
    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int ch = blockIdx.x % a.nch, bh = blockIdx.x / a.nch;
    const int b = bh / a.H, h = bh % a.H;
    const int t0 = ch * C, nval = min(C, a.N - t0);
    const RowView qv{(const char *)a.q + (b * a.sqb + h * a.sqh) * ES, a.sqn * ES, (a.N - 1) * a.sqn * ES + D * ES};
    const RowView kv{(const char *)a.k + (b * a.skb + h * a.skh) * ES, a.skn * ES, (a.N - 1) * a.skn * ES + D * ES};
    const RowView ov{(const char *)(a.out + b * a.sob + h * a.soh), a.son * 4, (a.N - 1) * a.son * 4 + D * 4};
    const RowView dov{(const char *)(a.dout + b * a.sdb + h * a.sdh), a.sdn * 4, (a.N - 1) * a.sdn * 4 + D * 4};
    // this lane's out row pieces and S_c pieces, requested with the stage
    const int t = 16 * w + r;
    const float *sc = a.fwd + ((int64_t)bh * a.P * a.NS + ch) * SL + DV * D;   // S_c (column block 0)
    const rsrc_t orow = ov.at(t0 + t, t < nval);
    f32x4 o4v[KT], s4v[KT];
#pragma unroll
    for (int js = 0; js < KT; ++js) {
        o4v[js] = __builtin_bit_cast(f32x4, bload16(orow, (uint32_t)((16 * js + 4 * g) * 4)));
        s4v[js] = *reinterpret_cast<const f32x4 *>(sc + 16 * js + 4 * g);
    }
    bwd_stage<F32, D, 1>(qv.at(t0), qv.rs, Gs, nval, tid);
    bwd_stage<F32, D, 1>(kv.at(t0), kv.rs, Fs, nval, tid);
    bwd_stage<true, D, 0>(dov.at(t0), dov.rs, Ns, nval, tid);
    __syncthreads();

    // ---- normaliser of token t = 16 w + r: g_t . (S_c + sum_{s <= t} f_s) + eps.
    // F becomes its inclusive prefix over the chunk's rows in place: NSEG
    // segments of rows per column, each summed by one thread, then offset by
    // the totals of the segments before it
    {
        constexpr int NSEG = NTHR / D, SEG = C / NSEG;
        const int j = tid % D, sg = tid / D;
        float run = 0.f;
#pragma unroll
        for (int i = 0; i < SEG; ++i) {
            run += Fs[(sg * SEG + i) * LD + j];
            Fs[(sg * SEG + i) * LD + j] = run;
        }
        __syncthreads();
        float off = 0.f;
#pragma unroll
        for (int s2 = 0; s2 < NSEG - 1; ++s2) off += s2 < sg ? Fs[(s2 * SEG + SEG - 1) * LD + j] : 0.f;
        __syncthreads();
#pragma unroll
        for (int i = 0; i < SEG; ++i) Fs[(sg * SEG + i) * LD + j] += off;
        __syncthreads();
    }
    float gs = 0.f, dot = 0.f;
#pragma unroll
    for (int js = 0; js < KT; ++js) {
        const f32x4 gq = nat4(Gs + t * LD + 16 * js + 4 * g);
        const f32x4 s4 = s4v[js] + nat4(Fs + t * LD + 16 * js + 4 * g), o4 = o4v[js];
        const f32x4 d4 = nat4(Ns + t * LD + 16 * js + 4 * g);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            gs += gq[i] * s4[i];
            dot += d4[i] * o4[i];
        }
    }
#pragma unroll
    for (int m = 16; m < WAVE; m <<= 1) {
        gs += __shfl_xor(gs, m);
        dot += __shfl_xor(dot, m);
    }
    const bool live = t < nval;
    const float den = gs + a.eps;
    const float ddn = live ? -dot / den : 0.f;
    const float inv = live ? 1.f / den : 0.f;
    if (g == 0) {
        dDs[t] = ddn;
        if (live) {
            a.den[(int64_t)bh * a.N + t0 + t] = den;
            a.dden[(int64_t)bh * a.N + t0 + t] = ddn;
        }
    }
    // dn_t = dout_t / D_t in place (lane (r, g) holds dims 16 js + 4g .. + 3)
#pragma unroll
    for (int js = 0; js < KT; ++js) {
        float *p = Ns + t * LD + 16 * js + 4 * g;
        *reinterpret_cast<f32x4 *>(p) = nat4(p) * inv;
    }
    __syncthreads();

    // ---- dR_c tiles (rows j, columns c), split over the waves
    float *slot0 = a.rev + ((int64_t)bh * a.P * a.NS + (a.nch - ch)) * SL;
    for (int tile = w; tile < KT * KT; tile += NWAVE) {
        const int jt = tile / KT, ct = tile % KT;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) acc = mma1(acc, trf(Gs, LD, 16 * ta, 16 * jt, r, g), trf(Ns, LD, 16 * ta, 16 * ct, r, g));
        const int c = 16 * ct + r;
        float *sl = slot0 + (int64_t)(c / DV) * a.NS * SL + c % DV;
#pragma unroll
        for (int i = 0; i < 4; ++i) sl[(16 * jt + 4 * g + i) * DV] = acc[i];
    }
    // ---- dr_c = sum_t g_t dD_t (NTHR / D partial sums per dim), into every
    // column block's slot
    {
        constexpr int NP = NTHR / D;
        const int j = tid % D, part = tid / D;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < C / NP; ++i) acc += Gs[(part + i * NP) * LD + j] * dDs[part + i * NP];
        red[tid] = acc;
        __syncthreads();
        if (tid < D) {
            float sum = 0.f;
#pragma unroll
            for (int pp = 0; pp < NP; ++pp) sum += red[pp * D + tid];
            for (int p = 0; p < a.P; ++p) slot0[(int64_t)p * a.NS * SL + DV * D + tid] = sum;
        }
    }
}

// dq, dk, dv of one chunk from the state before it, the adjoint state after
// it and the chunk's own tokens, every product on fp32 MFMA.  Wave w owns
// tokens 16 w .. + 15: their dq (as queries) and their dk, dv (as keys).
// Launched for fp32 inputs (bf16 inputs run k_bwd_chunk_bf).
template <bool F32, int D>
__global__ void __launch_bounds__(NTHR) k_bwd_chunk(const BwdArgs a)
{
    constexpr int C = 64, LD = D + 4, KT = D / 16, DV = D < 64 ? D : 64, SL = DV * D + D, ES = F32 ? 4 : 2;
    __shared__ __attribute__((aligned(16))) float sm[4 * C * LD + C];
    float *Gs = sm, *Fs = sm + C * LD, *Vs = sm + 2 * C * LD, *Ns = sm + 3 * C * LD, *dDs = sm + 4 * C * LD;
    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int ch = blockIdx.x % a.nch, bh = blockIdx.x / a.nch;
    const int b = bh / a.H, h = bh % a.H;
    const int t0 = ch * C, nval = min(C, a.N - t0);
    const RowView qv{(const char *)a.q + (b * a.sqb + h * a.sqh) * ES, a.sqn * ES, (a.N - 1) * a.sqn * ES + D * ES};
    const RowView kv{(const char *)a.k + (b * a.skb + h * a.skh) * ES, a.skn * ES, (a.N - 1) * a.skn * ES + D * ES};
    const RowView vv{(const char *)a.v + (b * a.svb + h * a.svh) * ES, a.svn * ES, (a.N - 1) * a.svn * ES + D * ES};
    const RowView dov{(const char *)(a.dout + b * a.sdb + h * a.sdh), a.sdn * 4, (a.N - 1) * a.sdn * 4 + D * 4};
    const float *denc = a.den + (int64_t)bh * a.N + t0;
    bwd_stage<F32, D, 1>(qv.at(t0), qv.rs, Gs, nval, tid);
    bwd_stage<F32, D, 1>(kv.at(t0), kv.rs, Fs, nval, tid);
    bwd_stage<F32, D, 0>(vv.at(t0), vv.rs, Vs, nval, tid);
    bwd_stage<true, D, 2>(dov.at(t0), dov.rs, Ns, nval, tid, denc);
    if (tid < C) dDs[tid] = tid < nval ? a.dden[(int64_t)bh * a.N + t0 + tid] : 0.f;
    __syncthreads();

    const int me = 16 * w + r;   // this lane's token (query for dq, key for dk / dv)
    const bool live = me < nval;
    // the state before the chunk (Z_c, S_c) and the adjoint state after it
    // (R', r'), column block p at + p * NS * SL
    const float *zc = a.fwd + ((int64_t)bh * a.P * a.NS + ch) * SL;
    const float *rc = a.rev + ((int64_t)bh * a.P * a.NS + (a.nch - 1 - ch)) * SL;
    auto zrow4 = [&](const float *st, int j, int c0) {   // st[j][c0 .. c0 + 3]
        return *reinterpret_cast<const f32x4 *>(st + (int64_t)(c0 / DV) * a.NS * SL + j * DV + c0 % DV);
    };

    // ---- dq (query me): rows j = 16 jt + 4g + i, column me
    {
        f32x4 acc[KT];
        const float ddt = dDs[me];
#pragma unroll
        for (int jt = 0; jt < KT; ++jt) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cs = 0; cs < KT; ++cs)
                x = mma1(x, zrow4(zc, 16 * jt + r, 16 * cs + 4 * g), nat4(Ns + me * LD + 16 * cs + 4 * g));
            const f32x4 s4 = *reinterpret_cast<const f32x4 *>(zc + DV * D + 16 * jt + 4 * g);
            acc[jt] = x + s4 * ddt;
        }
#pragma unroll
        for (int sa = 0; sa < 4; ++sa) {
            if (sa > w) break;
            f32x4 at = {0.f, 0.f, 0.f, 0.f};   // A^T: keys 16 sa + 4g + i, query me
#pragma unroll
            for (int cs = 0; cs < KT; ++cs)
                at = mma1(at, nat4(Vs + (16 * sa + r) * LD + 16 * cs + 4 * g), nat4(Ns + me * LD + 16 * cs + 4 * g));
#pragma unroll
            for (int i = 0; i < 4; ++i) at[i] = (16 * sa + 4 * g + i <= me) ? at[i] + ddt : 0.f;
#pragma unroll
            for (int jt = 0; jt < KT; ++jt) acc[jt] = mma1(acc[jt], trf(Fs, LD, 16 * sa, 16 * jt, r, g), at);
        }
        float *dst = a.dq + b * a.gqb + h * a.gqh + (int64_t)(t0 + me) * a.gqn;
        if (live) {
#pragma unroll
            for (int jt = 0; jt < KT; ++jt) {
                const f32x4 gq = nat4(Gs + me * LD + 16 * jt + 4 * g);
                f32x4 dphi;
#pragma unroll
                for (int i = 0; i < 4; ++i) dphi[i] = fminf(gq[i], 1.f);
                *reinterpret_cast<f32x4 *>(dst + 16 * jt + 4 * g) = acc[jt] * dphi;
            }
        }
    }
    // ---- dk (key me): rows j, column me
    {
        f32x4 acc[KT];
#pragma unroll
        for (int jt = 0; jt < KT; ++jt) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int cs = 0; cs < KT; ++cs)
                x = mma1(x, zrow4(rc, 16 * jt + r, 16 * cs + 4 * g), nat4(Vs + me * LD + 16 * cs + 4 * g));
            acc[jt] = x + *reinterpret_cast<const f32x4 *>(rc + DV * D + 16 * jt + 4 * g);
        }
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
            if (ta < w) continue;
            f32x4 at = {0.f, 0.f, 0.f, 0.f};   // A: queries 16 ta + 4g + i, key me
#pragma unroll
            for (int cs = 0; cs < KT; ++cs)
                at = mma1(at, nat4(Ns + (16 * ta + r) * LD + 16 * cs + 4 * g), nat4(Vs + me * LD + 16 * cs + 4 * g));
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tq = 16 * ta + 4 * g + i;
                at[i] = tq >= me ? at[i] + dDs[tq] : 0.f;
            }
#pragma unroll
            for (int jt = 0; jt < KT; ++jt) acc[jt] = mma1(acc[jt], trf(Gs, LD, 16 * ta, 16 * jt, r, g), at);
        }
        float *dst = a.dk + b * a.gkb + h * a.gkh + (int64_t)(t0 + me) * a.gkn;
        if (live) {
#pragma unroll
            for (int jt = 0; jt < KT; ++jt) {
                const f32x4 fk = nat4(Fs + me * LD + 16 * jt + 4 * g);
                f32x4 dphi;
#pragma unroll
                for (int i = 0; i < 4; ++i) dphi[i] = fminf(fk[i], 1.f);
                *reinterpret_cast<f32x4 *>(dst + 16 * jt + 4 * g) = acc[jt] * dphi;
            }
        }
    }
    // ---- dv: rows s = 16 w + 4g + i, columns c = 16 ct + r
    {
        f32x4 acc[KT];
#pragma unroll
        for (int ct = 0; ct < KT; ++ct) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            const int c = 16 * ct + r;
            const float *rcol = rc + (int64_t)(c / DV) * a.NS * SL + c % DV;
#pragma unroll
            for (int js = 0; js < KT; ++js) {
                f32x4 rb;   // R'[16 js + 4g + i][c]
#pragma unroll
                for (int i = 0; i < 4; ++i) rb[i] = rcol[(16 * js + 4 * g + i) * DV];
                x = mma1(x, nat4(Fs + me * LD + 16 * js + 4 * g), rb);
            }
            acc[ct] = x;
        }
#pragma unroll
        for (int ta = 0; ta < 4; ++ta) {
            if (ta < w) continue;
            f32x4 pt = {0.f, 0.f, 0.f, 0.f};   // P: queries 16 ta + 4g + i, key me
#pragma unroll
            for (int js = 0; js < KT; ++js)
                pt = mma1(pt, nat4(Gs + (16 * ta + r) * LD + 16 * js + 4 * g), nat4(Fs + me * LD + 16 * js + 4 * g));
#pragma unroll
            for (int i = 0; i < 4; ++i) pt[i] = (16 * ta + 4 * g + i >= me) ? pt[i] : 0.f;
#pragma unroll
            for (int ct = 0; ct < KT; ++ct) acc[ct] = mma1(acc[ct], pt, trf(Ns, LD, 16 * ta, 16 * ct, r, g));
        }
        float *dst = a.dv + b * a.gvb + h * a.gvh + (int64_t)t0 * a.gvn;
#pragma unroll
        for (int ct = 0; ct < KT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s = 16 * w + 4 * g + i;
                if (s < nval) dst[(int64_t)s * a.gvn + 16 * ct + r] = acc[ct][i];
            }
    }
}

// Stage 64 rows (a chunk) of one head into two swizzled bf16 [64][D] arrays:
// the values rounded to bf16 (hi) and the remainders (lo), hi + lo carrying
// about 16 significant bits; `lo2`, when given, gets a third part (about 24
// bits in all).  MODE 1: phi of bf16 inputs; MODE 2: fp32 inputs times
// 1 / den[row].  Both zero from row `nval` on.
template <int D, int MODE>
__device__ __forceinline__ void bwd_stage_split(rsrc_t src, int64_t rs, bf16 *hi, bf16 *lo, int nval, int tid,
                                                const float *den = nullptr, bf16 *lo2 = nullptr)
{
    constexpr int PPR = D / 8, ITEMS = 64 * PPR, NI = ITEMS / NTHR;   // 8-element pieces
    static_assert(ITEMS % NTHR == 0, "whole pieces per thread");
    float f[NI][8];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
        const int item = tid + it * NTHR, row = item / PPR, pc = item % PPR;
        if constexpr (MODE == 1) {
            Vec<false>::to_float(bload16(src, (uint32_t)(row * rs + pc * 16)), f[it]);
        } else {
            Vec<true>::to_float(bload16(src, (uint32_t)(row * rs + pc * 32)), f[it]);
            Vec<true>::to_float(bload16(src, (uint32_t)(row * rs + pc * 32 + 16)), f[it] + 4);
        }
    }
#pragma unroll
    for (int it = 0; it < NI; ++it) {
        const int item = tid + it * NTHR, row = item / PPR, pc = item % PPR;
        const bool live = row < nval;
        const float scale = MODE == 2 ? (live ? 1.f / den[row] : 0.f) : 1.f;
        u32x4 h, l, l2;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float x0 = f[it][2 * e], x1 = f[it][2 * e + 1];
            if constexpr (MODE == 1) { x0 = live ? phi<false>(x0) : 0.f; x1 = live ? phi<false>(x1) : 0.f; }
            else { x0 *= scale; x1 *= scale; }
            const uint2 s_ = split_pk(x0, x1);
            h[e] = s_.x;
            l[e] = s_.y;
            // third part: what hi + lo leave (hi + lo + lo2 carry about 24 bits)
            l2[e] = pk_bf16(x0 - bf_lo(s_.x) - bf_lo(s_.y), x1 - bf_hi(s_.x) - bf_hi(s_.y));
        }
        *reinterpret_cast<u32x4 *>(hi + swz<D>(row, pc * 8)) = h;
        *reinterpret_cast<u32x4 *>(lo + swz<D>(row, pc * 8)) = l;
        if (lo2) *reinterpret_cast<u32x4 *>(lo2 + swz<D>(row, pc * 8)) = l2;
    }
}

// k_bwd_chunk for bf16 inputs: the same gradients, every product on bf16
// MFMA (v_mfma_f32_16x16x32_bf16) with fp32 operands split into hi + lo
// (three products: hi hi, hi lo, lo hi).  G, F and dn are staged as hi + lo;
// v rows are read from memory.  v . dn, where v is exact, takes a third part
// of dn (about 24 bits in all): in A_ts = v_s . dn_t + dD_t the two terms
// cancel to the eps level at a head's first token (out_0 = v_0 up to eps),
// and the 16-bit hi + lo of dn left errors near 2e-3 of the row scale there.  Products contract
// either over dims / value columns (operands read as rows) or over tokens in
// steps of 32, in the token order t(g, j) = s0 + 4g + (j & 3) + 16 (j >> 2):
// then the two 16-token accumulator tiles at s0 and s0 + 16 are, lane by
// lane, the 8 operand values of the next product, and the other operand is a
// transpose read of a staged [token][dim] array.  The dq and dk tiles hold
// dims in the state tile order cs_dim (rows 4g .. 4g + 3 of tile jt are the
// consecutive dims 32 (jt >> 1) + 8g + 4 (jt & 1) + i), the layout of the
// transposed G and F operands; the state products read Z_c and R'_c rows in
// the same order.
template <int D>
__global__ void __launch_bounds__(NTHR) k_bwd_chunk_bf(const BwdArgs a)
{
    constexpr int C = 64, JT = D / 16, KS = D / 32, DV = D < 64 ? D : 64, SL = DV * D + D;
    // SH: Z_c and then R'_c are split once per workgroup into a shared
    // [D][D] hi + lo pair (d <= 64: 16 KB more LDS), instead of by every wave
    constexpr bool SH = D <= 64;
    __shared__ __attribute__((aligned(16))) bf16 sm[7 * C * D + (SH ? 2 * D * D : 0)];
    __shared__ float dDs[C];
    bf16 *Gh = sm, *Gl = sm + C * D, *Fh = sm + 2 * C * D, *Fl = sm + 3 * C * D;
    bf16 *Nh = sm + 4 * C * D, *Nl = sm + 5 * C * D, *Nl2 = sm + 6 * C * D, *Th = sm + 7 * C * D, *Tl = Th + D * D;
    const int tid = threadIdx.x, lane = tid % WAVE, r = lane % 16, g = lane / 16;
    const int w = __builtin_amdgcn_readfirstlane(tid / WAVE);
    const int ch = blockIdx.x % a.nch, bh = blockIdx.x / a.nch;
    const int b = bh / a.H, h = bh % a.H;
    const int t0 = ch * C, nval = min(C, a.N - t0);
    const RowView qv{(const char *)a.q + (b * a.sqb + h * a.sqh) * 2, a.sqn * 2, (a.N - 1) * a.sqn * 2 + D * 2};
    const RowView kv{(const char *)a.k + (b * a.skb + h * a.skh) * 2, a.skn * 2, (a.N - 1) * a.skn * 2 + D * 2};
    const RowView vv{(const char *)a.v + (b * a.svb + h * a.svh) * 2, a.svn * 2, (a.N - 1) * a.svn * 2 + D * 2};
    const RowView dov{(const char *)(a.dout + b * a.sdb + h * a.sdh), a.sdn * 4, (a.N - 1) * a.sdn * 4 + D * 4};
    const float *denc = a.den + (int64_t)bh * a.N + t0;
    bwd_stage_split<D, 1>(qv.at(t0), qv.rs, Gh, Gl, nval, tid);
    bwd_stage_split<D, 1>(kv.at(t0), kv.rs, Fh, Fl, nval, tid);
    // v rows are read from memory (L2) as operands: rows past the sequence
    // read as zeros
    const rsrc_t vr = vv.at(t0);
    auto vrow8 = [&](int row, int col) { return __builtin_bit_cast(bf16x8, bload16(vr, (uint32_t)(row * vv.rs + col * 2))); };
    bwd_stage_split<D, 2>(dov.at(t0), dov.rs, Nh, Nl, nval, tid, denc, Nl2);
    if (tid < C) dDs[tid] = tid < nval ? a.dden[(int64_t)bh * a.N + t0 + tid] : 0.f;
    __syncthreads();

    const int me = 16 * w + r;   // this lane's token (query for dq, key for dk / dv)
    const bool live = me < nval;
    const float *zc = a.fwd + ((int64_t)bh * a.P * a.NS + ch) * SL;
    const float *rc = a.rev + ((int64_t)bh * a.P * a.NS + (a.nch - 1 - ch)) * SL;
    auto zrow4 = [&](const float *st, int j, int c0) {   // st[j][c0 .. c0 + 3]
        return *reinterpret_cast<const f32x4 *>(st + (int64_t)(c0 / DV) * a.NS * SL + j * DV + c0 % DV);
    };
    auto dim0 = [&](int jt) { return 32 * (jt >> 1) + 8 * g + 4 * (jt & 1); };   // first dim of a lane's rows
    auto stage_state = [&](const float *st) {   // st[j][c] split into Th, Tl (swizzled [D][D])
        constexpr int PPR = D / 8, NI = D * PPR / NTHR > 0 ? D * PPR / NTHR : 1;
#pragma unroll
        for (int it = 0; it < NI; ++it) {
            const int item = tid + it * NTHR;
            if (item < D * PPR) {
                const int j = item / PPR, c8 = (item % PPR) * 8;
                bf16x8 hi, lo;
                cs_split(zrow4(st, j, c8), zrow4(st, j, c8 + 4), hi, lo);
                *reinterpret_cast<bf16x8 *>(Th + swz<D>(j, c8)) = hi;
                *reinterpret_cast<bf16x8 *>(Tl + swz<D>(j, c8)) = lo;
            }
        }
    };
    auto val4 = [&](const bf16 *hi, const bf16 *lo, int row, int col) {   // hi + lo of 4 staged values
        const uint2 x = *reinterpret_cast<const uint2 *>(hi + swz<D>(row, col));
        const uint2 y = *reinterpret_cast<const uint2 *>(lo + swz<D>(row, col));
        return (f32x4){bf_lo(x.x) + bf_lo(y.x), bf_hi(x.x) + bf_hi(y.x), bf_lo(x.y) + bf_lo(y.y), bf_hi(x.y) + bf_hi(y.y)};
    };

    if constexpr (SH) {
        stage_state(zc);
        __syncthreads();
    }
    // ---- dq (query me)
    {
        f32x4 acc[JT];
        const float ddt = dDs[me];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            const int jr = cs_dim(jt, r);
#pragma unroll
            for (int u = 0; u < KS; ++u) {
                bf16x8 zh, zl;
                if constexpr (SH) {
                    zh = nat8(Th + swz<D>(jr, 32 * u + 8 * g));
                    zl = nat8(Tl + swz<D>(jr, 32 * u + 8 * g));
                } else {
                    cs_split(zrow4(zc, jr, 32 * u + 8 * g), zrow4(zc, jr, 32 * u + 8 * g + 4), zh, zl);
                }
                const bf16x8 nh = nat8(Nh + swz<D>(me, 32 * u + 8 * g)), nl = nat8(Nl + swz<D>(me, 32 * u + 8 * g));
                x = mma8(x, zh, nh);
                x = mma8(x, zh, nl);
                x = mma8(x, zl, nh);
            }
            acc[jt] = x + *reinterpret_cast<const f32x4 *>(zc + DV * D + dim0(jt)) * ddt;
        }
        for (int v = 0; v <= (w >> 1); ++v) {   // keys up to the wave's last token
            const int s0 = 32 * v;
            f32x4 at[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4 t = {0.f, 0.f, 0.f, 0.f};   // v_s . dn_me, s = s0 + 16 hf + 4g + i
#pragma unroll
                for (int u = 0; u < KS; ++u) {
                    const bf16x8 va = vrow8(s0 + 16 * hf + r, 32 * u + 8 * g);
                    t = mma8(t, va, nat8(Nh + swz<D>(me, 32 * u + 8 * g)));
                    t = mma8(t, va, nat8(Nl + swz<D>(me, 32 * u + 8 * g)));
                    t = mma8(t, va, nat8(Nl2 + swz<D>(me, 32 * u + 8 * g)));
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) t[i] = (s0 + 16 * hf + 4 * g + i <= me) ? t[i] + ddt : 0.f;
                at[hf] = t;
            }
            bf16x8 bh_, bl_;
            cs_split(at[0], at[1], bh_, bl_);
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const bf16x8 fh = cs_ktr8<D>(Fh, s0, jt, r, g), fl = cs_ktr8<D>(Fl, s0, jt, r, g);
                acc[jt] = mma8(acc[jt], fh, bh_);
                acc[jt] = mma8(acc[jt], fh, bl_);
                acc[jt] = mma8(acc[jt], fl, bh_);
            }
        }
        if (live) {
            float *dst = a.dq + b * a.gqb + h * a.gqh + (int64_t)(t0 + me) * a.gqn;
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const f32x4 gq = val4(Gh, Gl, me, dim0(jt));
                f32x4 dphi;
#pragma unroll
                for (int i = 0; i < 4; ++i) dphi[i] = fminf(gq[i], 1.f);
                *reinterpret_cast<f32x4 *>(dst + dim0(jt)) = acc[jt] * dphi;
            }
        }
    }
    if constexpr (SH) {
        __syncthreads();   // every wave is done with Z_c
        stage_state(rc);
        __syncthreads();
    }
    // ---- dk (key me)
    {
        f32x4 acc[JT];
#pragma unroll
        for (int jt = 0; jt < JT; ++jt) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            const int jr = cs_dim(jt, r);
#pragma unroll
            for (int u = 0; u < KS; ++u) {
                bf16x8 rh, rl;
                if constexpr (SH) {
                    rh = nat8(Th + swz<D>(jr, 32 * u + 8 * g));
                    rl = nat8(Tl + swz<D>(jr, 32 * u + 8 * g));
                } else {
                    cs_split(zrow4(rc, jr, 32 * u + 8 * g), zrow4(rc, jr, 32 * u + 8 * g + 4), rh, rl);
                }
                const bf16x8 vb = vrow8(me, 32 * u + 8 * g);
                x = mma8(x, rh, vb);
                x = mma8(x, rl, vb);
            }
            acc[jt] = x + *reinterpret_cast<const f32x4 *>(rc + DV * D + dim0(jt));
        }
        for (int v = w >> 1; v < 2; ++v) {   // queries from the wave's first token on
            const int s0 = 32 * v;
            f32x4 at[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4 t = {0.f, 0.f, 0.f, 0.f};   // dn_t . v_me, t = s0 + 16 hf + 4g + i
#pragma unroll
                for (int u = 0; u < KS; ++u) {
                    const bf16x8 vb = vrow8(me, 32 * u + 8 * g);
                    t = mma8(t, nat8(Nh + swz<D>(s0 + 16 * hf + r, 32 * u + 8 * g)), vb);
                    t = mma8(t, nat8(Nl + swz<D>(s0 + 16 * hf + r, 32 * u + 8 * g)), vb);
                    t = mma8(t, nat8(Nl2 + swz<D>(s0 + 16 * hf + r, 32 * u + 8 * g)), vb);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tq = s0 + 16 * hf + 4 * g + i;
                    t[i] = tq >= me ? t[i] + dDs[tq] : 0.f;
                }
                at[hf] = t;
            }
            bf16x8 bh_, bl_;
            cs_split(at[0], at[1], bh_, bl_);
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const bf16x8 gh = cs_ktr8<D>(Gh, s0, jt, r, g), gl = cs_ktr8<D>(Gl, s0, jt, r, g);
                acc[jt] = mma8(acc[jt], gh, bh_);
                acc[jt] = mma8(acc[jt], gh, bl_);
                acc[jt] = mma8(acc[jt], gl, bh_);
            }
        }
        if (live) {
            float *dst = a.dk + b * a.gkb + h * a.gkh + (int64_t)(t0 + me) * a.gkn;
#pragma unroll
            for (int jt = 0; jt < JT; ++jt) {
                const f32x4 fk = val4(Fh, Fl, me, dim0(jt));
                f32x4 dphi;
#pragma unroll
                for (int i = 0; i < 4; ++i) dphi[i] = fminf(fk[i], 1.f);
                *reinterpret_cast<f32x4 *>(dst + dim0(jt)) = acc[jt] * dphi;
            }
        }
    }
    // ---- dv: rows s = 16 w + 4g + i (keys), columns c = 16 ct + r
    {
        f32x4 acc[JT];
#pragma unroll
        for (int ct = 0; ct < JT; ++ct) {
            f32x4 x = {0.f, 0.f, 0.f, 0.f};
            const int c = 16 * ct + r;
            const float *rcol = rc + (int64_t)(c / DV) * a.NS * SL + c % DV;
#pragma unroll
            for (int u = 0; u < KS; ++u) {
                if constexpr (SH) {
                    // dims in the transpose read's order 32u + 4g + (jj & 3) + 16 (jj >> 2)
                    const bf16x8 rh = tr8<D>(Th, 32 * u, 16 * ct, r, g), rl = tr8<D>(Tl, 32 * u, 16 * ct, r, g);
                    auto frow = [&](const bf16 *base) {
                        const bf16x4 x0 = *reinterpret_cast<const bf16x4 *>(base + swz<D>(16 * w + r, 32 * u + 4 * g));
                        const bf16x4 x1 = *reinterpret_cast<const bf16x4 *>(base + swz<D>(16 * w + r, 32 * u + 16 + 4 * g));
                        return __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
                    };
                    const bf16x8 fh = frow(Fh), fl = frow(Fl);
                    x = mma8(x, fh, rh);
                    x = mma8(x, fh, rl);
                    x = mma8(x, fl, rh);
                } else {
                    f32x4 r0, r1;   // R'[32u + 8g + jj][c]
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        r0[i] = rcol[(32 * u + 8 * g + i) * DV];
                        r1[i] = rcol[(32 * u + 8 * g + 4 + i) * DV];
                    }
                    bf16x8 rh, rl;
                    cs_split(r0, r1, rh, rl);
                    const bf16x8 fh = nat8(Fh + swz<D>(16 * w + r, 32 * u + 8 * g)), fl = nat8(Fl + swz<D>(16 * w + r, 32 * u + 8 * g));
                    x = mma8(x, fh, rh);
                    x = mma8(x, fh, rl);
                    x = mma8(x, fl, rh);
                }
            }
            acc[ct] = x;
        }
        for (int v = w >> 1; v < 2; ++v) {   // queries from the wave's first key on
            const int s0 = 32 * v;
            f32x4 pt[2];
#pragma unroll
            for (int hf = 0; hf < 2; ++hf) {
                f32x4 t = {0.f, 0.f, 0.f, 0.f};   // g_t . f_s, t = s0 + 16 hf + 4g + i, s = 16 w + r
#pragma unroll
                for (int u = 0; u < KS; ++u) {
                    const bf16x8 gh = nat8(Gh + swz<D>(s0 + 16 * hf + r, 32 * u + 8 * g));
                    const bf16x8 gl = nat8(Gl + swz<D>(s0 + 16 * hf + r, 32 * u + 8 * g));
                    const bf16x8 fh = nat8(Fh + swz<D>(me, 32 * u + 8 * g)), fl = nat8(Fl + swz<D>(me, 32 * u + 8 * g));
                    t = mma8(t, gh, fh);
                    t = mma8(t, gh, fl);
                    t = mma8(t, gl, fh);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) t[i] = (s0 + 16 * hf + 4 * g + i >= me) ? t[i] : 0.f;
                pt[hf] = t;
            }
            bf16x8 ph, pl;   // P^T rows s = 16 w + r over t(g, j)
            cs_split(pt[0], pt[1], ph, pl);
#pragma unroll
            for (int ct = 0; ct < JT; ++ct) {
                const bf16x8 nh = tr8<D>(Nh, s0, 16 * ct, r, g), nl = tr8<D>(Nl, s0, 16 * ct, r, g);
                acc[ct] = mma8(acc[ct], ph, nh);
                acc[ct] = mma8(acc[ct], ph, nl);
                acc[ct] = mma8(acc[ct], pl, nh);
            }
        }
        float *dst = a.dv + b * a.gvb + h * a.gvh + (int64_t)t0 * a.gvn;
#pragma unroll
        for (int ct = 0; ct < JT; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int s_ = 16 * w + 4 * g + i;
                if (s_ < nval) dst[(int64_t)s_ * a.gvn + 16 * ct + r] = acc[ct][i];
            }
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

// Columns per workgroup: at most 64 (two column blocks per head at d = 128).
inline int cols_per_wg(int d) { return d < 64 ? d : 64; }

template <bool F32, int D, int DV, int C>
constexpr bool fits() { return lds_bytes(F32, D, DV, C) <= LDS_LIMIT; }

// Chunk of 64 or 128 tokens (requests below 64 run as 64; fp32 inputs and
// d = 128 use 64: register budget).
int pick_chunk(bool f32, int d, int chunk)
{
    if (chunk == 0 || chunk < 64 || f32) chunk = 64;   // fp32: 64 (register budget)
    if (chunk >= 128 && d <= 64 && lds_bytes(f32, d, cols_per_wg(d), 128) <= LDS_LIMIT) return 128;
    return 64;
}

struct Plan {
    int C, DV, P, G, L, NS;
    size_t slot_floats;
    size_t part_bytes, fin_off, fin_bytes, flags_off, total;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Token groups: enough workgroups to cover the chip, each group a whole
// number of chunks, at most MAX_GROUPS groups per head.
constexpr int MAX_GROUPS = 32;
constexpr int CAUSAL_TARGET_WGS = 512;
// The last group of a causal call reads the slots of all earlier groups of its
// (head, column block): at most this many bytes.
constexpr size_t LOOKBACK_BYTES = 256 * 1024;
// A causal workspace starts with a status block: the 32-bit count of flag
// waits that gave up, at byte offset 0.  The slots and flags follow it.
constexpr size_t STATUS_BYTES = 256;
int pick_groups(int64_t units, int N, int C, int target, int max_groups = MAX_GROUPS)
{
    if (N <= 0) return 1;
    int64_t maxg = (N + C - 1) / C;
    int64_t g = (target + units - 1) / units;
    if (g < 1) g = 1;
    if (g > maxg) g = maxg;
    if (g > max_groups) g = max_groups;
    return (int)g;
}

void set_groups(Plan &pl, int N)
{
    int64_t per = (N + pl.G - 1) / pl.G;
    pl.L = (int)(((per + pl.C - 1) / pl.C) * pl.C);
    if (pl.L < pl.C) pl.L = pl.C;
    pl.G = N > 0 ? (int)((N + pl.L - 1) / pl.L) : 1;
}

// Single-pass causal plan (calls with outputs): G token groups per (head,
// column block), one slot and one flag per group, after the status block.
Plan plan_causal(int B, int H, int N, int d, la_dtype dt, int chunk)
{
    Plan pl;
    pl.C = pick_chunk(dt == LA_F32, d, chunk);
    pl.DV = cols_per_wg(d);
    pl.P = d / pl.DV;
    const int64_t BH = (int64_t)B * H;
    pl.slot_floats = (size_t)pl.DV * d + d;
    int max_g = 1 + (int)(LOOKBACK_BYTES / (pl.slot_floats * 4));
    // the column-split kernel at d = 128 holds 2 chunks per group: allow the
    // 16 groups that give it a full grid
    if (dt == LA_BF16 && d == 128 && pl.C == 64 && max_g < 16) max_g = 16;
    pl.G = pick_groups(BH * pl.P, N, pl.C, CAUSAL_TARGET_WGS, max_g < MAX_GROUPS ? max_g : MAX_GROUPS);
    set_groups(pl, N);
    pl.NS = N > 0 ? pl.G : 0;
    pl.part_bytes = pl.G > 1 ? align256((size_t)BH * pl.P * pl.G * pl.slot_floats * 4) : 0;
    pl.fin_off = STATUS_BYTES + pl.part_bytes;
    pl.fin_bytes = 0;
    pl.flags_off = STATUS_BYTES + pl.part_bytes;
    pl.total = N > 0 ? pl.flags_off + align256((size_t)BH * pl.P * pl.G * 8) : 0;
    return pl;
}

// A 64-bit tag unique to each call (splitmix64 of a per-process sequence):
// a flag counts as set only when it holds the tag of the running call, so the
// workspace needs no clearing between calls.
unsigned long long next_epoch()
{
    static std::atomic<unsigned long long> seq{(unsigned long long)time(nullptr) * 0x9E3779B97F4A7C15ull ^
                                               ((unsigned long long)getpid() << 32) ^ (uintptr_t)&seq};
    unsigned long long z = seq.fetch_add(0x9E3779B97F4A7C15ull) + 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    z ^= z >> 31;
    z &= ~0xfull;   // the low 4 bits of a flag carry the XCD index
    return z ? z : 16;
}

Plan plan_noncausal(int B, int H, int N, int d, la_dtype dt, int target = 1024)
{
    Plan pl;
    pl.C = pick_chunk(dt == LA_F32, d, 0);
    pl.DV = cols_per_wg(d);
    pl.P = d / pl.DV;
    const int64_t BH = (int64_t)B * H;
    pl.G = pick_groups(BH * pl.P, N, pl.C, target);
    set_groups(pl, N);
    pl.NS = pl.G;
    pl.slot_floats = (size_t)pl.DV * d + d;
    pl.part_bytes = align256((size_t)BH * pl.P * pl.NS * pl.slot_floats * 4);
    pl.fin_off = pl.part_bytes;
    pl.fin_bytes = align256((size_t)BH * pl.P * pl.slot_floats * 4);
    pl.flags_off = pl.fin_off + pl.fin_bytes;
    pl.total = N > 0 ? pl.fin_off + pl.fin_bytes : 0;
    return pl;
}

// State-only causal calls (out = NULL, the prefill): the non-causal partial
// states of the token shares, then their sum added to the carried-in state.
// Fewer, longer shares than the non-causal plan: the published states are
// then small next to k and v (B4 H8 N4096 d64: 14.2 us with about 256
// workgroups, 21.2 us with 1024, 19.2 us with 128).
constexpr int PREFILL_TARGET_WGS = 256;
Plan plan_state(int B, int H, int N, int d, la_dtype dt)
{
    Plan pl = plan_noncausal(B, H, N, d, dt, PREFILL_TARGET_WGS);
    pl.fin_bytes = 0;
    pl.total = N > 0 ? pl.part_bytes : 0;
    return pl;
}

// ---- kernel dispatch tables (dtype x d x chunk)
template <bool F32, int D, int C>
void launch_dc(int what, const Args &a, int nwg, hipStream_t st)
{
    constexpr int DV = D < 64 ? D : 64;
    if constexpr (fits<F32, D, DV, C>() && (C == 64 || (!F32 && D <= 64))) {
        if (what == 0) hipLaunchKernelGGL((k_group_state<F32, D, DV, C>), dim3(nwg), dim3(NTHR), 0, st, a);
        else if (what == 1) hipLaunchKernelGGL((k_chunk_fwd<F32, D, DV, C, MODE_OUT, 0>), dim3(nwg), dim3(NTHR), 0, st, a);
        else if (what == 2) hipLaunchKernelGGL((k_chunk_fwd<F32, D, DV, C, MODE_APPLY, 0>), dim3(nwg), dim3(NTHR), 0, st, a);
        else if constexpr (C == 64)
            hipLaunchKernelGGL((k_chunk_fwd<F32, D, DV, C, MODE_OUT, res_cpg(F32, D)>), dim3(nwg), dim3(NTHR), 0, st, a);
    }
}

template <bool F32, int D>
void dispatch_c(int C, int what, const Args &a, int nwg, hipStream_t st)
{
    // what: 0 = group state, 1 = causal with output, 2 = non-causal apply,
    // 3 = causal state only, 4 = causal with output, register-resident groups
    if (C == 128) launch_dc<F32, D, 128>(what, a, nwg, st);
    else launch_dc<F32, D, 64>(what, a, nwg, st);
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

// mode: 0 = scan into group starting states, 1 = total into z_out/s_out,
// 2 = total into fin, 3 = carried-in state into fin and total into z_out/s_out.
void launch_slots(int d, const Args &a, int64_t BH, int P, int nslots, int mode, hipStream_t st)
{
    const int sl = cols_per_wg(d) * d + d;
    dim3 grid((sl + 255) / 256, (unsigned)(BH * P));
    if (d == 32) hipLaunchKernelGGL((k_slots<32, 32>), grid, dim3(256), 0, st, a, nslots, mode);
    else if (d == 64) hipLaunchKernelGGL((k_slots<64, 64>), grid, dim3(256), 0, st, a, nslots, mode);
    else hipLaunchKernelGGL((k_slots<128, 64>), grid, dim3(256), 0, st, a, nslots, mode);
}

// column-split non-causal kernels (bf16, d = 64 or 128)
void launch_cs_state(int d, const Args &a, unsigned nwg, hipStream_t st)
{
    if (d == 64) hipLaunchKernelGGL((k_cs_state<64>), dim3(nwg), dim3(NTHR), 0, st, a);
    else hipLaunchKernelGGL((k_cs_state<128>), dim3(nwg), dim3(NTHR), 0, st, a);
}
void launch_cs_apply(int d, const Args &a, unsigned nwg, hipStream_t st)
{
    if (d == 64) hipLaunchKernelGGL((k_cs_apply<64>), dim3(nwg), dim3(NTHR), 0, st, a);
    else hipLaunchKernelGGL((k_cs_apply<128>), dim3(nwg), dim3(NTHR), 0, st, a);
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

// ---- scratch memory of la_causal_fwd_noalloc: one array per GPU, held by the
// code object until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device array: the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)32 << 20;
static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex scratch_mu;
void *scratch_addr[MAX_DEVICES];

// the current device's scratch address (nullptr if it cannot be resolved)
void *device_scratch()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(scratch_mu);
    if (!scratch_addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) {
            (void)hipGetLastError();
            return nullptr;
        }
        scratch_addr[dev] = p;
    }
    return scratch_addr[dev];
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
    case LA_ERR_UNSUPPORTED:
        return "LA_ERR_UNSUPPORTED: d must be 32, 64 or 128 and chunk 0, 16, 32, 64 or 128, and a causal call "
               "with outputs cannot be captured into a HIP graph";
    case LA_ERR_VALUE: return "LA_ERR_VALUE: eps must be finite and >= 0";
    case LA_ERR_WORKSPACE: return "LA_ERR_WORKSPACE: workspace missing or too small";
    case LA_ERR_ALIAS: return "LA_ERR_ALIAS: output state overlaps an input state";
    case LA_ERR_LAUNCH: return "LA_ERR_LAUNCH: a HIP launch failed";
    }
    return "unknown la_status";
}

int la_version(void) { return 100; }

size_t la_causal_fwd_workspace(int B, int H, int N, int d, int chunk)
{
    if (check_common(B, H, N, d, LA_BF16, 0.f) != LA_OK) return 0;
    if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return 0;
    // the largest plan over both dtypes, with and without outputs
    size_t total = 0;
    for (la_dtype dt : {LA_F32, LA_BF16}) {
        total = std::max(total, plan_causal(B, H, N, d, dt, chunk).total);
        total = std::max(total, plan_state(B, H, N, d, dt).total);
    }
    return total;
}

}  // extern "C"

namespace {
// ---- backward pass: workspace = forward slots, adjoint slots (nch + 1 per
// head and column block each), then D_t and dD_t per token
struct BwdPlan {
    int nch, DV, P, NS;
    size_t SL, slots_bytes, den_off, dden_off, total;
};
BwdPlan plan_bwd(int B, int H, int N, int d)
{
    BwdPlan pl;
    pl.nch = (N + 63) / 64;
    pl.DV = cols_per_wg(d);
    pl.P = d / pl.DV;
    pl.NS = pl.nch + 1;
    pl.SL = (size_t)pl.DV * d + d;
    const int64_t BH = (int64_t)B * H;
    pl.slots_bytes = align256((size_t)BH * pl.P * pl.NS * pl.SL * 4);
    pl.den_off = 2 * pl.slots_bytes;
    pl.dden_off = pl.den_off + align256((size_t)BH * N * 4);
    pl.total = N > 0 ? pl.dden_off + align256((size_t)BH * N * 4) : 0;
    return pl;
}

// bytes from p to one past the last element of a [B, H, N, d] tensor
size_t extent(la_strides s, int B, int H, int N, int d, size_t es)
{
    if (B == 0 || H == 0 || N == 0) return 0;
    return ((size_t)(B - 1) * s.b + (size_t)(H - 1) * s.h + (size_t)(N - 1) * s.n + d) * es;
}

// Memory calls run one segment at a time (a few thousand tokens per head):
// fewer, longer token groups than the non-causal plan, so that a group's
// published state does not outweigh its inputs, and shorter apply
// workgroups, so that the readout still covers the chip.
constexpr int MEM_GROUP_TARGET = 128;
constexpr int MEM_APPLY_CHUNKS = 2;
Plan plan_memory(int B, int H, int N, int d, la_dtype dt) { return plan_noncausal(B, H, N, d, dt, MEM_GROUP_TARGET); }

la_status causal_impl(const void *q, la_strides sq, const void *k, la_strides sk,
                      const void *v, la_strides sv, la_dtype dt,
                      float *out, la_strides so,
                      int B, int H, int N, int d, int chunk, float eps,
                      const float *z_in, const float *s_in,
                      float *z_out, float *s_out,
                      void *workspace, size_t ws_bytes, void *hip_stream, int unnorm,
                      bool use_scratch = false)
{
    la_status st = check_common(B, H, N, d, dt, eps);
    if (st != LA_OK) return st;
    if (chunk != 0 && chunk != 16 && chunk != 32 && chunk != 64 && chunk != 128) return LA_ERR_UNSUPPORTED;
    const size_t es = dt == LA_F32 ? 4 : 2;
    const bool want_out = out != nullptr;
    if (!want_out && !z_out && !s_out) return LA_ERR_NULL;
    if (N > 0) {
        // a state-only call reads k and v only
        if (want_out && (st = check_tensor(q, sq, es)) != LA_OK) return st;
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
    Plan pl = want_out ? plan_causal(B, H, N, d, dt, chunk) : plan_state(B, H, N, d, dt);
    if (ws_bytes < pl.total || (pl.total > 0 && !workspace && !use_scratch)) return LA_ERR_WORKSPACE;
    if (BH == 0) return LA_OK;
    if (use_scratch && pl.total > 0 && !(workspace = device_scratch())) return LA_ERR_LAUNCH;

    hipStream_t stream = (hipStream_t)hip_stream;
    (void)hipGetLastError();
    Args a = make_args(q, sq, k, sk, v, sv, out, so, B, H, N, eps);
    a.z_in = z_in; a.s_in = s_in; a.z_out = z_out; a.s_out = s_out;
    a.unnorm = unnorm;
    a.P = pl.P; a.L = pl.L; a.NS = pl.NS; a.G = pl.G;
    const bool f32 = dt == LA_F32;

    if (N == 0) {
        // the carried-in state (or zeros) passes through
        launch_slots(d, a, BH, pl.P, 0, 1, stream);
        return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
    }
    if (!want_out) {
        // prefill: the partial states of the token shares (k and v only),
        // then z_out = z_in + their sum in share order (each state element
        // read and written by one thread, so in place is safe)
        a.part = (float *)workspace;
        a.slot0 = 0;
        const unsigned nwg = (unsigned)(BH * pl.P * pl.G);
        if (!f32 && (d == 64 || d == 128) && pl.C == 64) {
            // one share per head and column block: the state kernel writes
            // the final state itself (no slots, no second launch)
            a.direct = pl.G == 1;
            launch_cs_state(d, a, nwg, stream);
            if (a.direct) return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
        } else {
            dispatch(f32, d, pl.C, 0, a, (int)nwg, stream);
        }
        launch_slots(d, a, BH, pl.P, pl.G, 1, stream);
        return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
    }
    // the look-back's tag is fixed here, so a captured graph would replay it
    {
        hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
        const hipError_t e = hipStreamIsCapturing(stream, &cap);
        (void)hipGetLastError();
        if ((e == hipSuccess && cap != hipStreamCaptureStatusNone) || e == hipErrorStreamCaptureImplicit)
            return LA_ERR_UNSUPPORTED;
    }
    a.giveups = (unsigned *)workspace;
    a.part = (float *)((char *)workspace + STATUS_BYTES);
    a.flags = (unsigned long long *)((char *)workspace + pl.flags_off);
    a.epoch = next_epoch();
    a.wait_tag = a.epoch;
    a.spin_limit = SPIN_LIMIT;
    // test hook: every wait looks for a tag that no workgroup stores and
    // gives up after the given number of polls (the kernels still end)
    if (const char *e = getenv("LA_TEST_LOOKBACK_TIMEOUT")) {
        const int n = atoi(e);
        if (n > 0) { a.wait_tag = a.epoch ^ 0x10ull; a.spin_limit = n; }
    }
    a.wait_s = (s_out && s_out == s_in && pl.P > 1) ? 1 : 0;
    const bool resident = pl.C == 64 && pl.L <= res_cpg(f32, d) * pl.C;
    const int nwg = (int)(BH * pl.P * pl.G);
#define LA_CS(DD, UN) hipLaunchKernelGGL((k_cs_fwd<DD, res_cpg(false, DD), UN>), dim3(nwg), dim3(NTHR), 0, stream, a)
    if (resident && !f32 && d == 64) {
        if (unnorm) LA_CS(64, true); else LA_CS(64, false);
    } else if (resident && !f32 && d == 128) {
        if (unnorm) LA_CS(128, true); else LA_CS(128, false);
    }
#undef LA_CS
    else
        dispatch(f32, d, pl.C, resident ? 4 : 1, a, nwg, stream);
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}
}  // namespace

extern "C" {

la_status la_causal_fwd(const void *q, la_strides sq, const void *k, la_strides sk,
                        const void *v, la_strides sv, la_dtype dt,
                        float *out, la_strides so,
                        int B, int H, int N, int d, int chunk, float eps,
                        const float *z_in, const float *s_in,
                        float *z_out, float *s_out,
                        void *workspace, size_t ws_bytes, void *hip_stream)
{
    return causal_impl(q, sq, k, sk, v, sv, dt, out, so, B, H, N, d, chunk, eps, z_in, s_in, z_out, s_out,
                       workspace, ws_bytes, hip_stream, 0);
}

la_status la_causal_fwd_noalloc(const void *q, la_strides sq, const void *k, la_strides sk,
                                const void *v, la_strides sv, la_dtype dt,
                                float *out, la_strides so,
                                int B, int H, int N, int d, int chunk, float eps,
                                const float *z_in, const float *s_in,
                                float *z_out, float *s_out, void *hip_stream)
{
    // the sizes whose workspace (as la_causal_fwd_workspace states it) fits
    if (la_causal_fwd_workspace(B, H, N, d, chunk) > NOALLOC_SCRATCH_BYTES) return LA_ERR_WORKSPACE;
    return causal_impl(q, sq, k, sk, v, sv, dt, out, so, B, H, N, d, chunk, eps, z_in, s_in, z_out, s_out,
                       nullptr, NOALLOC_SCRATCH_BYTES, hip_stream, 0, true);
}

size_t la_noalloc_scratch_bytes(void) { return NOALLOC_SCRATCH_BYTES; }

la_status la_causal_fwd_unnormalized(const void *q, la_strides sq, const void *k, la_strides sk,
                                     const void *v, la_strides sv, la_dtype dt,
                                     float *out, la_strides so,
                                     int B, int H, int N, int d, int chunk, float eps,
                                     const float *z_in, const float *s_in,
                                     float *z_out, float *s_out,
                                     void *workspace, size_t ws_bytes, void *hip_stream)
{
    return causal_impl(q, sq, k, sk, v, sv, dt, out, so, B, H, N, d, chunk, eps, z_in, s_in, z_out, s_out,
                       workspace, ws_bytes, hip_stream, 1);
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

size_t la_noncausal_workspace(int B, int H, int N, int d)
{
    if (check_common(B, H, N, d, LA_BF16, 0.f) != LA_OK) return 0;
    return std::max(plan_noncausal(B, H, N, d, LA_F32).total, plan_noncausal(B, H, N, d, LA_BF16).total);
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
    a.P = pl.P; a.NS = pl.NS;
    a.part = (float *)ws;
    a.fin = (float *)(ws + pl.fin_off);
    const bool f32 = dt == LA_F32;
    // 1) partial states of the token groups, 2) their sum per head in group
    // order, 3) every query against the global state
    a.G = pl.G; a.L = pl.L; a.slot0 = 0;
    const bool cs = !f32 && (d == 64 || d == 128) && pl.C == 64;
    if (cs) launch_cs_state(d, a, (unsigned)(BH * pl.P * pl.G), stream);
    else dispatch(f32, d, pl.C, 0, a, (int)(BH * pl.P * pl.G), stream);
    launch_slots(d, a, BH, pl.P, pl.G, 2, stream);
    const int la = pl.C * 4;
    a.L = la;
    a.G = (N + la - 1) / la;
    if (cs) launch_cs_apply(d, a, (unsigned)(BH * pl.P * a.G), stream);
    else dispatch(f32, d, pl.C, 2, a, (int)(BH * pl.P * a.G), stream);
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

size_t la_causal_bwd_workspace(int B, int H, int N, int d)
{
    if (check_common(B, H, N, d, LA_BF16, 0.f) != LA_OK) return 0;
    return plan_bwd(B, H, N, d).total;
}

la_status la_causal_bwd(const void *q, la_strides sq, const void *k, la_strides sk,
                        const void *v, la_strides sv, la_dtype dt,
                        const float *out, la_strides so, const float *dout, la_strides sdo,
                        int B, int H, int N, int d, float eps,
                        const float *z_in, const float *s_in, const float *dz_out, const float *ds_out,
                        float *dq, la_strides sdq, float *dk, la_strides sdk, float *dv, la_strides sdv,
                        float *dz_in, float *ds_in,
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
        if ((st = check_tensor(dout, sdo, 4)) != LA_OK) return st;
        if ((st = check_tensor(dq, sdq, 4)) != LA_OK) return st;
        if ((st = check_tensor(dk, sdk, 4)) != LA_OK) return st;
        if ((st = check_tensor(dv, sdv, 4)) != LA_OK) return st;
    }
    for (const void *p : {(const void *)z_in, (const void *)s_in, (const void *)dz_out, (const void *)ds_out,
                          (const void *)dz_in, (const void *)ds_in})
        if (p && !aligned16(p)) return LA_ERR_ALIGN;
    const int64_t BH = (int64_t)B * H;
    const size_t zb = (size_t)BH * d * d * 4, sb = (size_t)BH * d * 4;
    // the gradients overlap no input and no other gradient
    {
        const void *ins[] = {q, k, v, out, dout, z_in, s_in, dz_out, ds_out};
        const size_t in_n[] = {extent(sq, B, H, N, d, es), extent(sk, B, H, N, d, es), extent(sv, B, H, N, d, es),
                               extent(so, B, H, N, d, 4), extent(sdo, B, H, N, d, 4), zb, sb, zb, sb};
        void *outs[] = {dq, dk, dv, dz_in, ds_in};
        const size_t out_n[] = {extent(sdq, B, H, N, d, 4), extent(sdk, B, H, N, d, 4), extent(sdv, B, H, N, d, 4),
                                zb, sb};
        for (int i = 0; i < 5; ++i) {
            for (int j = 0; j < 9; ++j)
                if (overlaps(outs[i], out_n[i], ins[j], in_n[j])) return LA_ERR_ALIAS;
            for (int j = i + 1; j < 5; ++j)
                if (overlaps(outs[i], out_n[i], outs[j], out_n[j])) return LA_ERR_ALIAS;
        }
    }
    const BwdPlan pl = plan_bwd(B, H, N, d);
    if (ws_bytes < pl.total || (pl.total > 0 && !workspace)) return LA_ERR_WORKSPACE;
    if (BH == 0) return LA_OK;
    hipStream_t stream = (hipStream_t)hip_stream;
    (void)hipGetLastError();
    char *ws = (char *)workspace;
    const bool f32 = dt == LA_F32;
    // the slot kernels' view: (Z_c, S_c) slots, scans, totals
    Args a = make_args(q, sq, k, sk, v, sv, nullptr, la_strides{0, 0, 0}, B, H, N, eps);
    a.P = pl.P;
    a.NS = pl.NS;
    if (N == 0) {
        // no token: the gradient reaching the carried-in state is dz_out
        a.z_in = dz_out; a.s_in = ds_out; a.z_out = dz_in; a.s_out = ds_in;
        if (dz_in || ds_in) launch_slots(d, a, BH, pl.P, 0, 1, stream);
        return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
    }
    float *fwd = (float *)ws, *rev = (float *)(ws + pl.slots_bytes);
    // 1) the forward state before every chunk: chunk partial states into
    //    slots 1.., then the scan (slot c = state_in + chunks 0 .. c-1)
    a.part = fwd; a.G = pl.nch; a.L = 64; a.slot0 = 1;
    a.z_in = z_in; a.s_in = s_in;
    dispatch(f32, d, 64, 0, a, (int)(BH * pl.P * pl.nch), stream);
    launch_slots(d, a, BH, pl.P, pl.NS, 0, stream);
    // 2) normalisers and the chunks' adjoint parts (reverse-indexed slots)
    BwdArgs ba;
    memset(&ba, 0, sizeof(ba));
    ba.q = q; ba.k = k; ba.v = v; ba.out = out; ba.dout = dout;
    ba.sqb = sq.b; ba.sqh = sq.h; ba.sqn = sq.n; ba.skb = sk.b; ba.skh = sk.h; ba.skn = sk.n;
    ba.svb = sv.b; ba.svh = sv.h; ba.svn = sv.n; ba.sob = so.b; ba.soh = so.h; ba.son = so.n;
    ba.sdb = sdo.b; ba.sdh = sdo.h; ba.sdn = sdo.n;
    ba.dq = dq; ba.dk = dk; ba.dv = dv;
    ba.gqb = sdq.b; ba.gqh = sdq.h; ba.gqn = sdq.n; ba.gkb = sdk.b; ba.gkh = sdk.h; ba.gkn = sdk.n;
    ba.gvb = sdv.b; ba.gvh = sdv.h; ba.gvn = sdv.n;
    ba.B = B; ba.H = H; ba.N = N; ba.nch = pl.nch; ba.P = pl.P; ba.NS = pl.NS; ba.eps = eps;
    ba.fwd = fwd; ba.rev = rev;
    ba.den = (float *)(ws + pl.den_off); ba.dden = (float *)(ws + pl.dden_off);
    const dim3 grid((unsigned)(BH * pl.nch));
#define LA_BWD(KERN, F, DD) hipLaunchKernelGGL((KERN<F, DD>), grid, dim3(NTHR), 0, stream, ba)
    if (f32) {
        if (d == 32) LA_BWD(k_bwd_prep, true, 32); else if (d == 64) LA_BWD(k_bwd_prep, true, 64); else LA_BWD(k_bwd_prep, true, 128);
    } else {
        if (d == 32) LA_BWD(k_bwd_prep, false, 32); else if (d == 64) LA_BWD(k_bwd_prep, false, 64); else LA_BWD(k_bwd_prep, false, 128);
    }
    // 3) the gradient reaching the carried-in state: dz_out + every chunk's part
    a.z_in = dz_out; a.s_in = ds_out; a.z_out = dz_in; a.s_out = ds_in;
    if (dz_in || ds_in) {
        Args t = a;
        t.part = rev + pl.SL;   // slots 1 .. nch of every (head, column block)
        launch_slots(d, t, BH, pl.P, pl.nch, 1, stream);
    }
    // 4) the adjoint state after every chunk (slot nch - 1 - c)
    a.part = rev;
    launch_slots(d, a, BH, pl.P, pl.NS, 0, stream);
    // 5) dq, dk, dv of every chunk
    if (f32) {
        if (d == 32) LA_BWD(k_bwd_chunk, true, 32); else if (d == 64) LA_BWD(k_bwd_chunk, true, 64); else LA_BWD(k_bwd_chunk, true, 128);
    } else {
#define LA_BWD_BF(DD) hipLaunchKernelGGL((k_bwd_chunk_bf<DD>), grid, dim3(NTHR), 0, stream, ba)
        if (d == 32) LA_BWD_BF(32); else if (d == 64) LA_BWD_BF(64); else LA_BWD_BF(128);
#undef LA_BWD_BF
    }
#undef LA_BWD
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

size_t la_memory_workspace(int B, int H, int N, int d)
{
    if (check_common(B, H, N, d, LA_BF16, 0.f) != LA_OK) return 0;
    return std::max(plan_memory(B, H, N, d, LA_F32).total, plan_memory(B, H, N, d, LA_BF16).total);
}

// The non-causal kernels with the carried-in memory as the state that the
// queries read: 1) partial states of the segment's token groups, 2) the
// memory copied for the readout and the updated memory written out, 3) every
// query against the memory before the segment.
la_status la_memory_fwd(const void *q, la_strides sq, const void *k, la_strides sk,
                        const void *v, la_strides sv, la_dtype dt,
                        float *out, la_strides so,
                        int B, int H, int N, int d, float eps,
                        const float *z_in, const float *s_in,
                        float *z_out, float *s_out,
                        void *workspace, size_t ws_bytes, void *hip_stream)
{
    la_status st = check_common(B, H, N, d, dt, eps);
    if (st != LA_OK) return st;
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
    if (z_out && z_in && z_out != (float *)z_in && overlaps(z_out, zb, z_in, zb)) return LA_ERR_ALIAS;
    if (s_out && s_in && s_out != (float *)s_in && overlaps(s_out, sb, s_in, sb)) return LA_ERR_ALIAS;
    if (overlaps(z_out, zb, s_in, sb) || overlaps(s_out, sb, z_in, zb) || overlaps(z_out, zb, s_out, sb))
        return LA_ERR_ALIAS;
    Plan pl = plan_memory(B, H, N, d, dt);
    if (ws_bytes < pl.total || (pl.total > 0 && !workspace)) return LA_ERR_WORKSPACE;
    if (BH == 0) return LA_OK;
    hipStream_t stream = (hipStream_t)hip_stream;
    (void)hipGetLastError();
    char *ws = (char *)workspace;
    Args a = make_args(q, sq, k, sk, v, sv, out, so, B, H, N, eps);
    a.z_in = z_in; a.s_in = s_in; a.z_out = z_out; a.s_out = s_out;
    a.P = pl.P; a.NS = pl.NS;
    if (N == 0) {
        // the carried-in memory (or zeros) passes through
        launch_slots(d, a, BH, pl.P, 0, 1, stream);
        return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
    }
    a.part = (float *)ws;
    a.fin = want_out ? (float *)(ws + pl.fin_off) : nullptr;
    const bool f32 = dt == LA_F32;
    a.G = pl.G; a.L = pl.L; a.slot0 = 0;
    const bool cs = !f32 && (d == 64 || d == 128) && pl.C == 64;
    if (cs && want_out) {
        // one launch: the partial states and the reads of the memory (two
        // workgroups per share), then the memory after the segment
        const unsigned nwg = (unsigned)(2 * BH * pl.P * pl.G);
        if (d == 64) hipLaunchKernelGGL((k_cs_memory<64>), dim3(nwg), dim3(NTHR), 0, stream, a);
        else hipLaunchKernelGGL((k_cs_memory<128>), dim3(nwg), dim3(NTHR), 0, stream, a);
        launch_slots(d, a, BH, pl.P, pl.G, 1, stream);
        return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
    }
    if (cs) launch_cs_state(d, a, (unsigned)(BH * pl.P * pl.G), stream);
    else dispatch(f32, d, pl.C, 0, a, (int)(BH * pl.P * pl.G), stream);
    launch_slots(d, a, BH, pl.P, pl.G, 3, stream);
    if (want_out) {
        const int la = pl.C * MEM_APPLY_CHUNKS;
        a.L = la;
        a.G = (N + la - 1) / la;
        if (cs) launch_cs_apply(d, a, (unsigned)(BH * pl.P * a.G), stream);
        else dispatch(f32, d, pl.C, 2, a, (int)(BH * pl.P * a.G), stream);
    }
    return hipGetLastError() == hipSuccess ? LA_OK : LA_ERR_LAUNCH;
}

}  // extern "C"
