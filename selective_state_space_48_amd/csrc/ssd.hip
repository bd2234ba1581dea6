// Mamba-2's state space dual (SSD) layer on gfx950 matrix cores.
//
// The restricted selective SSM of the state space duality ("State Space
// Models Explained: How Mamba Works and How It Compares to Transformers"
// (mernstackdev.com), section "From S4 to Mamba"; "State space models and
// Mamba: reading long sequences without attention" (ai-trend.me), section
// "How it developed: from S4 to Mamba and Mamba-2"): one scalar decay
// a_t = exp(delta_t A_h) per token and head, heads of P channels, B and C
// shared by the heads. Per batch entry and head, with S the N x P state:
//     S_t = a_t S_{t-1} + delta_t B_t x_t^T,   y_t = C_t^T S_t + D_h x_t.
// Its dual is a masked matrix product, y = (L o C B^T)(delta x) + D x with
// L[t,s] = a_{s+1} ... a_t, a semiseparable matrix; cutting the sequence into
// chunks of Q tokens splits it into diagonal blocks (small dense products)
// and low-rank off-diagonal parts carried by the state between chunks. Per
// chunk, with cum_t the running sum of log2-decays inside the chunk and
// H the state entering it:
//   y_t   = sum_{s<=t} [C_t . B_s] 2^(cum_t - cum_s) delta_s x_s      (scores)
//         + 2^(cum_t) C_t^T H + D x_t                                  (carry-in)
//   H'    = 2^(cum_end) H + sum_s 2^(cum_end - cum_s) delta_s B_s x_s^T
// Every product is a v_mfma_f32_32x32x16_bf16: bf16 operands (the inputs,
// the masked and scaled scores, the scaled B and the carried state rounded
// to bf16 as operands), fp32 sums; the state itself is accumulated in fp32.
//
// One workgroup (4 waves) per (batch, head) walks the chunks in order and
// keeps the state in matrix-core accumulators, so no chunk state ever goes
// to HBM: x, delta, B and C are read once (B and C, shared by the heads, from
// L2 after the first head) and y is written once. Wave w owns the 32 x 32
// output tile (t block w/2, p block w%2) and the state tiles of p block w%2
// for half of the state rows. A wave's state rows stay in its accumulators
// from chunk to chunk (never in LDS): each wave forms C.H over its half of
// the state rows for both t blocks, and the two waves of a p block exchange
// those partial products (4 KB per wave) through LDS.
// Tiles are staged in LDS as the rows arrive (16-byte writes, no transposes):
// the operands whose contraction runs over tokens (x for the outputs, B and
// the weighted x for the state) are read with the LDS transpose read, and
// the masked scores have a tile of their own, so a chunk takes three
// barriers. The next chunk's inputs are loaded into registers while the
// current one computes, by whole 128-byte lines.
#include "common.hpp"
#include "launch.hpp"

namespace selscan {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));

constexpr int kQ = 64;   // tokens per chunk
constexpr int kP = 64;   // headdim

// acc[r] of a 32 x 32 MFMA tile is element (row, col) = (8*(r/4) + 4*(lane/32) + r%4, lane%32);
// operands: lane holds 8 consecutive K of row lane%32 (A) or column lane%32 (B), K offset 8*(lane/32).
__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r / 4) + 4 * (lane / 32) + r % 4; }
// 8 consecutive bf16 from LDS (16 bytes, aligned).
__device__ __forceinline__ bf16x8 lds8(const bf16_bits* p) {
    return *reinterpret_cast<const bf16x8*>(p);
}
__device__ __forceinline__ bf16_bits tobf(float v) { return from_f32<bf16_bits>(v); }
__device__ __forceinline__ float bfval(bf16_bits v) { return __uint_as_float(uint32_t(v) << 16); }
// The 8 bf16 of a 16-byte piece, in order.
__device__ __forceinline__ void split8(const uint4& v, bf16_bits* o) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        o[2 * k] = bf16_bits(w[k] & 0xffffu);
        o[2 * k + 1] = bf16_bits(w[k] >> 16);
    }
}

// Inclusive prefix sum over the 64 lanes of a wave: Hillis-Steele steps by
// DPP row shifts inside each row of 16 lanes (zero-filled), then the row
// totals carried across rows by the row broadcasts of lanes 15 and 31.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shifted(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL,
                                                                 ROW_MASK, 0xf, false));
}
__device__ __forceinline__ float wave_prefix_sum(float v) {
    v += dpp_shifted<0x111, 0xf>(v);  // row_shr:1
    v += dpp_shifted<0x112, 0xf>(v);  // row_shr:2
    v += dpp_shifted<0x114, 0xf>(v);  // row_shr:4
    v += dpp_shifted<0x118, 0xf>(v);  // row_shr:8
    v += dpp_shifted<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_shifted<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

struct SsdArgs {
    const bf16_bits* x;     // [batch, L, H, P]
    const bf16_bits* delta; // [batch, L, H]
    const float* A;         // [H]
    const bf16_bits* B;     // [batch, L, N]
    const bf16_bits* C;     // [batch, L, N]
    const float* D;         // [H] or null
    const float* dt_bias;   // [H] or null
    bf16_bits* y;           // [batch, L, H, P]
    float* last_state;      // [batch, H, N, P] or null
    const float* h0;        // [batch, H, N, P] state entering token 0, or null (zeros)
    int64_t batch, L, H;
};

// One chunk's inputs as this thread loads them. Wave wv loads tokens
// 16 wv .. 16 wv + 15 as whole rows, consecutive lanes on consecutive 16-byte
// pieces (every load instruction covers whole 128-byte lines): B and C piece
// k of token tokB(k), x piece k of token tokX(k); and the raw step of token
// lane, which every wave needs for its running decay.
template <int N>
struct ChunkRegs {
    static constexpr int NP = N / 8;      // 16-byte pieces of a B (or C) row
    static constexpr int NB = NP / 4;     // of them per thread
    uint4 b[NB], c[NB], x[2];
    float dl;
    bool ok;  // token lane exists (tokens past the end take step 0: an identity step)
    static __device__ __forceinline__ int tokB(int wv, int k, int lane) { return 16 * wv + k * (64 / NP) + lane / NP; }
    static __device__ __forceinline__ int tokX(int wv, int k, int lane) { return 16 * wv + 8 * k + lane / 8; }
};

// LDS tiles are stored row-major without padding; their 16-byte pieces are
// permuted within each row by an XOR with a function of the row, chosen so
// that every access of the kernel spreads over the banks (16-byte reads: 16
// lanes on distinct pieces mod 16; 8-byte and transposed reads: 32 lanes on
// distinct 8-byte units mod 32; 16-byte writes: 8 lanes on distinct pieces
// mod 8; 4-byte writes: 32 lanes on distinct words mod 32).
// Rows of 16 pieces (B and C, N = 128): any 16 consecutive rows differ mod 16,
// any 8 consecutive rows differ mod 8, and each aligned group of 4 rows puts a
// given 64-byte run into 4 different 64-byte bank ranges.
__device__ __forceinline__ int swz16(int r) {
    return ((r & 3) << 2) ^ (r & 3) ^ ((r >> 2) & 1) ^ (((r >> 3) & 1) << 1);
}
// Rows of 8 pieces (B and C for N = 64, x): 8 consecutive rows differ mod 8,
// even and odd rows each differ among any 8, and rows j, j + 2 of an aligned
// group of 4 land in different halves of the 32 banks.
__device__ __forceinline__ int swz8(int r) {
    const int m = (r >> 1) & 7;
    return (((m & 1) << 2) | ((m >> 1) & 3)) ^ ((r & 1) << 1);
}
// The masked scores [t][s]: 16-byte reads of 16 consecutive rows, and 4-byte
// writes that put rows R, R + 1 (R even) into different halves of the banks.
__device__ __forceinline__ int swzm(int r) { return ((r >> 1) & 7) ^ ((r & 1) << 2); }
// Element offset of (row, col) in a tile of NPR pieces per row.
template <int NPR>
__device__ __forceinline__ int at(int row, int col) {
    const int sw = NPR == 16 ? swz16(row) : swz8(row);
    return row * NPR * 8 + (((col >> 3) ^ sw) << 3) + (col & 7);
}
__device__ __forceinline__ int atm(int row, int col) {
    return row * kQ + (((col >> 3) ^ swzm(row)) << 3) + (col & 7);
}

// ds_read_b64_tr_b16: every lane reads 4 bf16 and the wave's 16-lane groups
// exchange them so that lane i receives element i % 4 of what lane
// 16 (i / 16) + 4 e + (i % 16) / 4 read, e = 0..3 (checked on gfx950). Lane
// (g = l / 16, j = l % 16 / 4, q = l % 4) reading row k0 + 8 (g / 2) + j at
// column c + 4 q therefore hands lane i the column of lane i's tile position
// at rows k0 + 8 (i / 32) + 0..3: half of a matrix-core operand whose
// contraction index runs down the rows of a row-major tile.
__device__ __forceinline__ bf16x4 ldtr(const bf16_bits* p) {
    typedef short s4 __attribute__((ext_vector_type(4)));
    const s4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) s4*)(const_cast<bf16_bits*>(p)));
    return __builtin_bit_cast(bf16x4, v);
}
// Operand (K = tile rows k0 .. k0 + 15, columns c0 .. c0 + 31) of a row-major
// tile of NPR pieces per row: lane l gets rows k0 + 8 (l / 32) + 0..7 of
// column c0 + perm(l % 32), perm swapping bits 2 and 3 when PERM is set.
template <int NPR, bool PERM>
__device__ __forceinline__ bf16x8 tr_operand(const bf16_bits* tile, int k0, int c0, int lane) {
    const int g = lane / 16, j = (lane % 16) / 4, q = lane % 4;
    const int qq = PERM ? (((q & 1) << 1) | (q >> 1)) : q;
    const int row = k0 + 8 * (g / 2) + j, col = c0 + 16 * (g % 2) + 4 * qq;
    const bf16x4 lo = ldtr(tile + at<NPR>(row, col));
    const bf16x4 hi = ldtr(tile + at<NPR>(row + 4, col));
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Raw buffer resource of `bytes` bytes at p (loads past the end read zeros,
// stores past it are dropped).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), short(0), bytes, 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int off) {
    return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// State rows are held in the accumulators in the order that makes the
// carry-in product's C operand one contiguous 16-byte read: accumulator row i
// of a 32-row tile is state row tau(i) (bits 2 and 3 swapped).
__device__ __forceinline__ int tau(int i) { return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1); }

template <int N>
__global__ __launch_bounds__(256, 2) void ssd_fused(SsdArgs a) {
    constexpr int NP = N / 8;        // 16-byte pieces per B/C row
    constexpr int NT = N / 32;       // 32-row tiles of the state
    constexpr int NTW = NT / 2;      // state tiles per wave
    using R = ChunkRegs<N>;
    __shared__ alignas(16) bf16_bits Cs[kQ * N];       // C rows [t][n]
    __shared__ alignas(16) bf16_bits Bs[kQ * N];       // B rows [s][n]
    __shared__ alignas(16) bf16_bits Xn[kQ * kP];      // x rows [s][p]
    __shared__ alignas(16) bf16_bits Xw[kQ * kP];      // 2^(cum_end - cum_s) delta_s x_s: [s][p]
    __shared__ alignas(16) bf16_bits Ms[kQ * kQ];      // masked scores [t][s]
    __shared__ alignas(16) float4 Yx[4][4][64];       // carry-in partial sums for the partner wave
    __shared__ float cums[kQ], dts[kQ], gcum[kQ];      // running log2-decay, step and 2^cum of the chunk's tokens

    const int tid = threadIdx.x, lane = tid % 64;
    const int wv = __builtin_amdgcn_readfirstlane(tid / 64);
    const int pb = wv % 2, tb = wv / 2;
    // The heads of a batch entry, which read the same B and C rows, run on one XCD (one L2).
    const int64_t bh = xcd_tile(blockIdx.x, gridDim.x);
    const int64_t b = bh / a.H, h = bh % a.H;
    const int nc = int((a.L + kQ - 1) / kQ);
    const float Ah = a.A[h] * kLog2e;                      // log2 decay per unit step
    const float bias = a.dt_bias ? a.dt_bias[h] : 0.0f;
    const float Dh = a.D ? a.D[h] : 0.0f;

    // Loads are unconditional (a token past the end reads the last token's
    // row: valid memory) so that they need no branches; staging zeroes such
    // tokens, whose step is 0 (an identity step).
    // Chunk loads and stores go through buffer resources based at the
    // chunk's first token and sized to its last valid one: a token past the
    // end reads zeros and its stores are dropped by the hardware's range
    // check, so the partial last chunk needs no guards. Lane offsets are
    // fixed; only the (scalar) resources change from chunk to chunk.
    const int64_t xs = a.H * kP;  // elements from one token's x (or y) row to the next
    int vB[R::NB], vX[2];
#pragma unroll
    for (int k = 0; k < R::NB; ++k) vB[k] = (R::tokB(wv, k, lane) * N + (lane % NP) * 8) * 2;
#pragma unroll
    for (int k = 0; k < 2; ++k) vX[k] = int((R::tokX(wv, k, lane) * xs + (lane % 8) * 8) * 2);
    const int vD = int(lane * a.H * 2);
    auto valid = [&](int c) { return int(min(int64_t(kQ), a.L - int64_t(c) * kQ)); };
    // Bytes from a chunk's first row to the end of the last valid row's
    // `row` elements, rows `stride` elements apart; 0 for a chunk past the
    // end (the prefetch after the last chunk), so that nothing is read.
    auto span = [](int nv, int64_t stride, int64_t row) { return nv > 0 ? int(((nv - 1) * stride + row) * 2) : 0; };
    auto load = [&](int c, R& r) {
        const int64_t t0 = int64_t(c) * kQ;
        const int nv = valid(c);
        r.ok = lane < nv;
        const auto rB = buf_rsrc(a.B + (b * a.L + t0) * N, span(nv, N, N));
        const auto rC = buf_rsrc(a.C + (b * a.L + t0) * N, span(nv, N, N));
        const auto rX = buf_rsrc(a.x + ((b * a.L + t0) * a.H + h) * kP, span(nv, xs, kP));
        const auto rD = buf_rsrc(a.delta + (b * a.L + t0) * a.H + h, span(nv, a.H, 1));
#pragma unroll
        for (int k = 0; k < R::NB; ++k) {
            r.b[k] = buf_load16(rB, vB[k]);
            r.c[k] = buf_load16(rC, vB[k]);
        }
#pragma unroll
        for (int k = 0; k < 2; ++k) r.x[k] = buf_load16(rX, vX[k]);
        r.dl = to_f32(bf16_bits(__builtin_amdgcn_raw_buffer_load_b16(rD, vD, 0, 0)));
    };

    // State tiles (fp32 accumulators), from h0 or zero: accumulator row i of
    // tile j is state row n = 32 (tb NTW + j) + tau(i), column p = 32 pb +
    // lane % 32. The wave keeps its own rows of the state for its p block
    // from chunk to chunk; the carry-in product C H is summed over n in two
    // halves, one per wave of the p block, which swap partial sums through LDS.
    f32x16 H[NTW];
    if (a.h0) {
        const float* src = a.h0 + (b * a.H + h) * int64_t(N) * kP;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                H[j][r] = src[int64_t((tb * NTW + j) * 32 + tau(acc_row(r, lane))) * kP + pb * 32 + lane % 32];
    } else {
#pragma unroll
        for (int j = 0; j < NTW; ++j) H[j] = f32x16{};
    }

    // A chunk's outputs are stored as soon as they are formed, after the
    // next chunk's loads were issued. Vector-memory waits count loads and
    // stores together in issue order, so the wait for those loads (at the
    // next chunk's staging) leaves the stores in flight.
    uint32_t ypend[8];  // two adjacent columns (bf16) for each pair of rows
    const int vY = int(((tb * 32 + 4 * (lane / 32) + (lane & 1)) * xs + pb * 32 + (lane % 32 & ~1)) * 2);
    auto store_y = [&](int c) {
        const int64_t t0 = int64_t(c) * kQ;
        const auto rY = buf_rsrc(a.y + ((b * a.L + t0) * a.H + h) * kP, span(valid(c), xs, kP));
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int dr = 8 * (k / 2) + 2 * (k % 2);  // rows dr and dr + 1 of the pair
            __builtin_amdgcn_raw_buffer_store_b32(ypend[k], rY, vY + int(dr * xs * 2), 0, 0);
        }
    };
    // Of each pair of rows (dr, dr + 1) held by a lane pair (columns s, s + 1),
    // the even lane keeps row dr and the odd lane row dr + 1, swapping one
    // value through a DPP quad permutation (lanes 0<->1, 2<->3); returns the
    // two adjacent columns of the lane's row, packed as bf16.
    auto pair_rows = [&](float v0, float v1) {
        const bool odd = lane & 1;
        const float send = odd ? v0 : v1;
        const float recv = __builtin_bit_cast(
            float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, send), 0xb1, 0xf, 0xf, false));
        return odd ? pack_bf16x2(recv, v1) : pack_bf16x2(v0, recv);
    };

    R cur;
    load(0, cur);
    // Zeros for the first chunk's outputs (overwritten by the same lanes in
    // the first iteration): the loop is then entered, like every back edge,
    // with 8 stores behind the loads of the chunk it starts with.
#pragma unroll
    for (int k = 0; k < 8; ++k) ypend[k] = 0;
    store_y(0);
    for (int c = 0; c < nc; ++c) {
        // Staging (and the stores and prefetch issued with it) runs at a
        // raised wave priority, the matrix products at the base one: the
        // other workgroup's waves on the same SIMDs then reach their next
        // chunk's products sooner.
        __builtin_amdgcn_s_setprio(1);
        // ---- per-token: step size and running log2-decay, token = lane (every wave) ----
        const float sp = softplus_log2(cur.dl + bias) * kLn2;
        const float dt = cur.ok ? sp : 0.0f;
        const float cum = wave_prefix_sum(dt * Ah);
        const float cend = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, cum), kQ - 1));
        // ---- stage chunk c: rows as loaded, 16-byte writes ----
        {
            const int s = lane;
            if (wv == 0) {
                gcum[s] = exp2_hw(cum);
                cums[s] = cum;
                dts[s] = dt;
            }
            const float ws_t = exp2_hw(cend - cum) * dt;  // weight of token s in the state update
#pragma unroll
            for (int k = 0; k < R::NB; ++k) {
                const int tok = R::tokB(wv, k, lane), col = (lane % NP) * 8;
                *reinterpret_cast<uint4*>(&Cs[at<NP>(tok, col)]) = cur.c[k];
                *reinterpret_cast<uint4*>(&Bs[at<NP>(tok, col)]) = cur.b[k];
            }
#pragma unroll
            for (int k = 0; k < 2; ++k) {
                const int tok = R::tokX(wv, k, lane), col = (lane % 8) * 8;
                const float ws = __shfl(ws_t, tok, 64);  // the weight of this piece's token
                const uint4 v = cur.x[k];
                *reinterpret_cast<uint4*>(&Xn[at<8>(tok, col)]) = v;
                uint4 w;
                w.x = pack_bf16x2(ws * bf16_lo(v.x), ws * bf16_hi(v.x));
                w.y = pack_bf16x2(ws * bf16_lo(v.y), ws * bf16_hi(v.y));
                w.z = pack_bf16x2(ws * bf16_lo(v.z), ws * bf16_hi(v.z));
                w.w = pack_bf16x2(ws * bf16_lo(v.w), ws * bf16_hi(v.w));
                *reinterpret_cast<uint4*>(&Xw[at<8>(tok, col)]) = w;
            }
        }
        load(c + 1, cur);  // next chunk's inputs, in flight during this chunk
        __syncthreads();
        __builtin_amdgcn_s_setprio(0);

        // ---- carry-in partials: C (both t blocks) times this wave's state rows ----
        // Registers 8 kb .. 8 kb + 7 of a state tile hold accumulator rows
        // 16 kb + 4 (lane / 32) + {0..3, 8..11}, i.e. state rows 16 kb +
        // 8 (lane / 32) + 0..7: as the B operand they pair with one 16-byte
        // piece of each C row.
        f32x16 Yp[2] = {f32x16{}, f32x16{}};
        {
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
#pragma unroll
                for (int kb = 0; kb < 2; ++kb) {
                    bf16x8 hb;
#pragma unroll
                    for (int e = 0; e < 8; ++e) hb[e] = __bf16(H[j][8 * kb + e]);
                    const int n0 = (tb * NTW + j) * 32 + 16 * kb + 8 * (lane / 32);
#pragma unroll
                    for (int tt = 0; tt < 2; ++tt)
                        Yp[tt] = mfma(lds8(&Cs[at<NP>(tt * 32 + lane % 32, n0)]), hb, Yp[tt]);
                }
            }
            // the partner wave (same p block, other t block) gets its tile's half
            const f32x16& give = Yp[1 - tb];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                Yx[pb * 2 + (1 - tb)][q][lane] =
                    make_float4(give[4 * q], give[4 * q + 1], give[4 * q + 2], give[4 * q + 3]);
        }

        // ---- scores of the lower block triangle: wave 0 (0,0), wave 1 (1,0), wave 2 (1,1) ----
        if (wv < 3) {
            const int gt = wv == 0 ? 0 : 1, gs = wv == 2 ? 1 : 0;
            f32x16 G = {};
#pragma unroll
            for (int ks = 0; ks < N / 16; ++ks) {
                const int k0 = ks * 16 + 8 * (lane / 32);
                G = mfma(lds8(&Cs[at<NP>(gt * 32 + lane % 32, k0)]), lds8(&Bs[at<NP>(gs * 32 + lane % 32, k0)]), G);
            }
            // Branch-free: every lane forms its 16 values and keeps those on
            // or below the diagonal (the exponent is clamped at 0 above it).
            const int s = gs * 32 + lane % 32;
            const float cs = cums[s], ds = dts[s];
            const int t0 = gt * 32 + 4 * (lane / 32);  // row of G[0]
            const float* crow = &cums[t0];
            float m[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dr = 8 * (r / 4) + r % 4;
                const float v = G[r] * exp2_hw(fminf(crow[dr] - cs, 0.0f)) * ds;
                m[r] = t0 + dr >= s ? v : 0.0f;
            }
            const int odd = lane & 1;
#pragma unroll
            for (int r = 0; r < 16; r += 2) {
                const int dr = 8 * (r / 4) + r % 4;
                *reinterpret_cast<uint32_t*>(&Ms[atm(t0 + dr + odd, s & ~1)]) = pair_rows(m[r], m[r + 1]);
            }
        }
        __syncthreads();

        // ---- output tile (tb, pb): scores x x  +  2^cum_t (C H)  +  D x ----
        {
            f32x16 y1 = {};
#pragma unroll
            for (int ks = 0; ks < kQ / 16; ++ks) {
                if (ks < 2 * (tb + 1)) {  // s blocks above the diagonal are all masked
                    const int k0 = ks * 16 + 8 * (lane / 32);
                    y1 = mfma(lds8(&Ms[atm(tb * 32 + lane % 32, k0)]), tr_operand<8, false>(Xn, ks * 16, pb * 32, lane), y1);
                }
            }
            // C H: this wave's half plus the partner's (written before the last barrier)
            f32x16 y2 = Yp[tb];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const float4 v = Yx[pb * 2 + tb][q][lane];
                y2[4 * q] += v.x; y2[4 * q + 1] += v.y; y2[4 * q + 2] += v.z; y2[4 * q + 3] += v.w;
            }
            const int p = pb * 32 + lane % 32;
            const int t0 = tb * 32 + 4 * (lane / 32);  // chunk row of y1[0]
            const float* grow = &gcum[t0];
            float v[16];
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int dr = 8 * (r / 4) + r % 4;
                v[r] = fmaf(grow[dr], y2[r], y1[r]) + Dh * bfval(Xn[at<8>(t0 + dr, p)]);
            }
            // Stores of two adjacent columns at once (rows paired as in the scores).
#pragma unroll
            for (int r = 0; r < 16; r += 2) ypend[r / 2] = pair_rows(v[r], v[r + 1]);
            store_y(c);
        }
        // ---- state: H <- 2^cum_end H + B^T (w x) over this wave's tiles ----
        {
            const float gend = exp2_hw(cend);
            bf16x8 xw[kQ / 16];
#pragma unroll
            for (int ks = 0; ks < kQ / 16; ++ks) xw[ks] = tr_operand<8, false>(Xw, ks * 16, pb * 32, lane);
#pragma unroll
            for (int j = 0; j < NTW; ++j) {
                const int nb = tb * NTW + j;
                f32x16 acc = H[j] * gend;
#pragma unroll
                for (int ks = 0; ks < kQ / 16; ++ks)
                    acc = mfma(tr_operand<NP, true>(Bs, ks * 16, nb * 32, lane), xw[ks], acc);
                H[j] = acc;
            }
        }
        __syncthreads();  // every read of this chunk's tiles is done
    }
    if (a.last_state) {
        float* dst = a.last_state + (b * a.H + h) * int64_t(N) * kP;
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r)
                dst[int64_t((tb * NTW + j) * 32 + tau(acc_row(r, lane))) * kP + pb * 32 + lane % 32] = H[j][r];
    }
}

struct SsdStepArgs {
    float* state;           // [batch, H, N, P], updated in place
    const bf16_bits* x;     // [batch, H, P]
    const bf16_bits* delta; // [batch, H]
    const float* A;         // [H]
    const bf16_bits* B;     // [batch, N]
    const bf16_bits* C;     // [batch, N]
    const float* D;         // [H] or null
    const float* dt_bias;   // [H] or null
    bf16_bits* y;           // [batch, H, P]
    int64_t H;
};

// One decode step of the layer: per (batch entry, head) the N x P state is
// read and written once (the step is bound by that traffic). Thread (nq, p4)
// takes the 4 channels 4 p4.. and the state rows n = nq + 16 k, so a wave
// moves four whole 256-byte rows per access; the readout's partial sums over
// n meet in LDS and are added in order.
template <int N>
__global__ __launch_bounds__(256) void ssd_step_kernel(SsdStepArgs a) {
    constexpr int K = N / 16;
    __shared__ float red[16][kP];
    const int tid = threadIdx.x, p4 = tid % 16, nq = tid / 16;
    const int64_t bh = blockIdx.x, b = bh / a.H, h = bh % a.H;
    const float l = softplus_log2(to_f32(a.delta[bh]) + (a.dt_bias ? a.dt_bias[h] : 0.0f));
    const float decay = exp2_hw(l * a.A[h]);  // exp(delta A), delta = l ln 2
    const float dl = l * kLn2;
    const uint2 xr = *reinterpret_cast<const uint2*>(a.x + bh * kP + 4 * p4);
    const float xs[4] = {bf16_lo(xr.x), bf16_hi(xr.x), bf16_lo(xr.y), bf16_hi(xr.y)};
    float* S = a.state + bh * int64_t(N) * kP + 4 * p4;
    f32x4v s[K];
#pragma unroll
    for (int k = 0; k < K; ++k)
        s[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4v*>(S + (nq + 16 * k) * kP));
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const int n = nq + 16 * k;
        const float u = dl * to_f32(a.B[b * N + n]), c = to_f32(a.C[b * N + n]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            s[k][i] = fmaf(decay, s[k][i], u * xs[i]);
            acc[i] = fmaf(c, s[k][i], acc[i]);
        }
        __builtin_nontemporal_store(s[k], reinterpret_cast<f32x4v*>(S + n * kP));
    }
    *reinterpret_cast<float4*>(&red[nq][4 * p4]) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (tid < kP) {
        float y = 0.0f;
#pragma unroll
        for (int q = 0; q < 16; ++q) y += red[q][tid];
        const float Dh = a.D ? a.D[h] : 0.0f;
        a.y[bh * kP + tid] = tobf(fmaf(Dh, to_f32(a.x[bh * kP + tid]), y));
    }
}

}  // namespace

hipError_t launch_ssd_step(const SsdStepTensors& t, int64_t batch, int64_t heads, int64_t dstate,
                           hipStream_t stream) {
    SsdStepArgs k{};
    k.state = t.state;
    k.x = static_cast<const bf16_bits*>(t.x);
    k.delta = static_cast<const bf16_bits*>(t.delta);
    k.A = t.A;
    k.B = static_cast<const bf16_bits*>(t.B);
    k.C = static_cast<const bf16_bits*>(t.C);
    k.D = t.D;
    k.dt_bias = t.dt_bias;
    k.y = static_cast<bf16_bits*>(t.y);
    k.H = heads;
    const dim3 grid(unsigned(batch * heads)), block(256);
    if (dstate == 64) hipLaunchKernelGGL((ssd_step_kernel<64>), grid, block, 0, stream, k);
    else hipLaunchKernelGGL((ssd_step_kernel<128>), grid, block, 0, stream, k);
    return hipGetLastError();
}

hipError_t launch_ssd(const SsdTensors& t, int64_t batch, int64_t L, int64_t heads, int64_t dstate,
                      hipStream_t stream) {
    SsdArgs k{};
    k.x = static_cast<const bf16_bits*>(t.x);
    k.delta = static_cast<const bf16_bits*>(t.delta);
    k.A = t.A;
    k.B = static_cast<const bf16_bits*>(t.B);
    k.C = static_cast<const bf16_bits*>(t.C);
    k.D = t.D;
    k.dt_bias = t.dt_bias;
    k.y = static_cast<bf16_bits*>(t.y);
    k.last_state = t.last_state;
    k.h0 = t.h0;
    k.batch = batch; k.L = L; k.H = heads;
    const dim3 grid(unsigned(batch * heads)), block(256);
    if (dstate == 64) hipLaunchKernelGGL((ssd_fused<64>), grid, block, 0, stream, k);
    else hipLaunchKernelGGL((ssd_fused<128>), grid, block, 0, stream, k);
    return hipGetLastError();
}

}  // namespace selscan
