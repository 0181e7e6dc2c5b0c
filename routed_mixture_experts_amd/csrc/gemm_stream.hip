// Weight-streaming grouped GEMMs of the routed-MoE forward on gfx950: groups of
// at most 64 rows (all of decode) and dense products with few rows.  The
// product is the one of gemm.hip ("vLLM-Ascend Kimi K3 MoE Forward Insight",
// Stage 4: grouped gate/up -> activation -> grouped down), with the weights
// as the streamed operand.
//  * gemm_bf16_stream -- each wave of an 8-wave workgroup streams 16 whole
//    weight rows straight into MFMA registers; the token rows come from an LDS
//    double buffer.
//  * gemm_bf16_stream_ksplit -- the same product with K split over 4 waves,
//    for dense products too small to fill the chip with whole-row streams.
#include "gemm_tiles.h"

namespace moe {

namespace {

using namespace tiles;

// ------------------------------------------------------------------------
// bf16 weight-streaming MFMA kernel (<= 64 rows per tile)
// ------------------------------------------------------------------------
constexpr int SROWS = 16;   // token rows per MFMA block (and per dense tile)
constexpr int SNW = 64;     // weight rows per workgroup

// One tile of up to 16*NB token rows: each wave streams its quarter of K for
// 64 weight rows and applies every weight fragment to all NB token blocks.
// SU k-steps (of 32) form one load batch; two batches are in flight.
template <int EPI, int NB, int SU>
__device__ __forceinline__ void stream_tile(const GemmArgs& g, const TileCoord& tc,
                                            float (*red)[4][4][64]) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, kofs = (lane >> 4) * 8;

    // 32-bit byte offsets from wave-uniform bases (one VGPR per row); every
    // operand of one group fits in 4 GiB (checked on the host)
    const char* Bb = (const char*)((const bf16_t*)g.B + (int64_t)tc.group * g.b_gstride);
    const char* B2b = (const char*)g.B2;
    const char* Ab = (const char*)g.A;
    const char* A2b = (const char*)g.A2;
    uint32_t wo[4], wo2[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        int wrow;
        if (SW) {
            const int c = min(tc.nt * 32 + (q & 1) * 16 + l16, g.N - 1);
            wrow = q < 2 ? c : g.N + c;
        } else {
            wrow = min(tc.nt * SNW + q * 16 + l16, g.N - 1);
        }
        wo[q] = (uint32_t)((int64_t)wrow * g.K * 2) + kofs * 2;
        wo2[q] = (uint32_t)((int64_t)wrow * g.K2 * 2) + kofs * 2;
    }
    uint32_t xo[NB], xo2[NB];
    bool xvalid[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        const int r = tc.row0 + tb * 16 + l16;
        xvalid[tb] = r < tc.row1;
        xo[tb] = (uint32_t)((xvalid[tb] ? a_row_of(g, r) : 0) * g.lda * 2) + kofs * 2;
        xo2[tb] = (uint32_t)((int64_t)(xvalid[tb] ? r : 0) * g.lda2 * 2) + kofs * 2;
    }

    const int ns1 = g.K / 32;
    const int ns = ns1 + (g.A2 ? g.K2 / 32 : 0);
    const int s0 = (int)((int64_t)wave * ns / 4), s1 = (int)((int64_t)(wave + 1) * ns / 4);

    f32x4_t acc[4][NB];
#pragma unroll
    for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) acc[q][tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    u32x4_t wa[SU][4], xa[SU][NB], wb[SU][4], xb[SU][NB];
    const u32x4_t zero = {0u, 0u, 0u, 0u};

    auto load = [&](int sbase, u32x4_t (&w)[SU][4], u32x4_t (&x)[SU][NB])
                    __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            const int st = sbase + u;
            if (st < s1) {
                if (st < ns1) {
                    const uint32_t ko = st * 64;
#pragma unroll
                    for (int q = 0; q < 4; ++q) w[u][q] = *(const u32x4_t*)(Bb + (wo[q] + ko));
#pragma unroll
                    for (int tb = 0; tb < NB; ++tb)
                        x[u][tb] = xvalid[tb] ? *(const u32x4_t*)(Ab + (xo[tb] + ko)) : zero;
                } else {
                    const uint32_t ko = (st - ns1) * 64;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        w[u][q] = *(const u32x4_t*)(B2b + (wo2[q] + ko));
#pragma unroll
                    for (int tb = 0; tb < NB; ++tb)
                        x[u][tb] = xvalid[tb] ? *(const u32x4_t*)(A2b + (xo2[tb] + ko)) : zero;
                }
            }
        }
    };
    auto compute = [&](int sbase, u32x4_t (&w)[SU][4], u32x4_t (&x)[SU][NB])
                       __attribute__((always_inline)) {
#pragma unroll
        for (int u = 0; u < SU; ++u) {
            if (sbase + u < s1) {
#pragma unroll
                for (int tb = 0; tb < NB; ++tb) {
                    const bf16x8_t xb8 = __builtin_bit_cast(bf16x8_t, x[u][tb]);
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        acc[q][tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, w[u][q]), xb8, acc[q][tb], 0, 0, 0);
                }
            }
        }
    };

    load(s0, wa, xa);
    for (int s = s0; s < s1; s += 2 * SU) {
        load(s + SU, wb, xb);
        compute(s, wa, xa);
        load(s + 2 * SU, wa, xa);
        compute(s + SU, wb, xb);
    }

    // acc[q][tb][j] holds C[weight row 4*(lane/16)+j of group q][token 16*tb + lane%16]
    const int wr = (lane >> 4) * 4;
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) {
        if (tb > 0) __syncthreads();
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int j = 0; j < 4; ++j) red[wave][q][j][lane] = acc[q][tb][j];
        __syncthreads();
        const int rr = tc.row0 + tb * 16 + l16;
        if (SW) {
            if (wave < 2) {
                const int q = wave;
                float gsum[4], usum[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    gsum[j] = red[0][q][j][lane] + red[1][q][j][lane] + red[2][q][j][lane] +
                              red[3][q][j][lane];
                    usum[j] = red[0][q + 2][j][lane] + red[1][q + 2][j][lane] +
                              red[2][q + 2][j][lane] + red[3][q + 2][j][lane];
                }
                if (rr < tc.row1) {
                    bf16_t* crow = (bf16_t*)g.C + (int64_t)rr * g.ldc;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int hc = tc.nt * 32 + q * 16 + wr + j;
                        if (hc < g.N) crow[hc] = f32_to_bf16(glu_f32(gsum[j], usum[j], g));
                    }
                }
            }
        } else {
            const int q = wave;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                v[j] = red[0][q][j][lane] + red[1][q][j][lane] + red[2][q][j][lane] +
                       red[3][q][j][lane];
            if (rr < tc.row1) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = tc.nt * SNW + q * 16 + wr + j;
                    if (c >= g.N) continue;
                    float o = v[j];
                    if (EPI == EPI_F32_BIAS && g.bias) o += g.bias[c];
                    if (EPI == EPI_OUT)
                        ((bf16_t*)g.C)[(int64_t)rr * g.ldc + c] = f32_to_bf16(o);
                    else
                        ((float*)g.C)[(int64_t)rr * g.ldc + c] = o;
                }
            }
        }
    }
}

// Dense products with few tiles: splitting K over the waves keeps more of
// the chip busy than whole-row streams would.
template <int EPI>
__global__ __launch_bounds__(256) void gemm_bf16_stream_ksplit(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    const int ntn = SW ? (g.N + 31) / 32 : (g.N + SNW - 1) / SNW;
    TileCoord tc;
    if (!fetch_tile(g, SROWS, ntn, tc)) return;
    __shared__ float red[4][4][4][64];
    const int rows = tc.row1 - tc.row0;
    if (rows <= 16) stream_tile<EPI, 1, 4>(g, tc, red);
    else if (rows <= 32) stream_tile<EPI, 2, 2>(g, tc, red);
    else stream_tile<EPI, 4, 2>(g, tc, red);
}


// Whole-row weight streams.  Each wave owns 16 weight rows (SwiGLU: 8 gate
// rows and the 8 up rows of the same hidden columns) over the full K, so
// every wave reads 16 long contiguous rows -- the pattern that keeps HBM
// near its streaming rate; splitting K over waves (four read positions per
// row) runs about 12% slower.  The token rows, shared by the 4 waves, come
// from LDS: chunks of CS k-steps are loaded a chunk ahead into registers
// (each wave a quarter of the chunk), written to a double buffer, and
// published with one barrier per chunk.  Weight fragments run PD k-steps
// ahead in registers.  Reading the token operand straight from global
// memory beside the weights costs up to a third of the bandwidth, which is
// why it is staged.  Every vector-memory operation here is a register load,
// so the compiler's in-order vmcnt bookkeeping stays exact (LDS-DMA loads
// mixed with register loads make it fall back to draining the counter).
// NW = 8 waves per workgroup, 16 weight rows each: SRN = 16 * NW weight rows
// per workgroup (SwiGLU: SRN / 2 columns), and a 64 KB token buffer.  (A
// 16-wave form, 256 weight rows per workgroup, streamed groups of 16 or more
// rows faster while the weights came in half-line loads; with whole-line
// load pairs 8 waves are faster at every group size measured.)
template <int NW>
constexpr int sx_bytes() { return NW * 8 * 1024; }

int stream_col_tiles_nw(int epi, int N, int nw) {
    const int srn = 16 * nw;
    return epi == EPI_SWIGLU ? (N + srn / 2 - 1) / (srn / 2) : (N + srn - 1) / srn;
}

// With FP8 weights (OCP e4m3 codes, one fp32 scale per weight row) each
// 16-byte weight load holds 16 codes, i.e. two 32-deep k-steps: lane g4 of a
// 64-deep block takes k 16*g4 .. +15, its first 8 for the even step and the
// rest for the odd one.  With MXFP4 weights (OCP E2M1 codes, two per byte,
// one E8M0 exponent per 32 codes of a row) a 16-byte load holds 32 codes --
// one scale block -- i.e. four k-steps.  K a multiple of 512: two loads
// take the 128 bytes of a 256-deep block of the wave's 16 rows as whole
// cache lines (8 rows each, 8 lanes a row), and a lane exchange gives lane
// l of row l % 16 the 64 codes k = 64*g4 .. +63 of the block, 8 per step
// (the memory instructions and cache lines of this stream, rather than its
// bytes, set its pace).  Otherwise lane g4 of a 128-deep block takes k
// 32*g4 .. +31, 8 per step, and the 4 block exponents of a load unit come
// in one dword beside it.  The token operand is staged with the same k order
// as the weights, the codes become bf16 exactly in registers (MXFP4: with
// the block scale applied by the conversion), and FP8's row scale multiplies
// the fp32 sums in the epilogue.
//
// A tile of at most 16 / QF rows (QF = 2 or 4, one token block) loads its
// token rows QF k-steps per 1 KB load instead of one: lane l takes row
// l % (16 / QF) and the 8 elements that operand lane l % (16 / QF) + 16 * g4
// of k-step l / (64 / QF) holds (g4 = (l / (16 / QF)) % 4), and writes them
// to that place of the same LDS blocks, so the MFMA side is unchanged.
// Operand rows past 16 / QF keep whatever the buffer held: they only feed
// output rows past the tile's end, which are never stored.  At decode most
// groups have at most 4 rows, and the token loads then take a quarter of
// the load slots.
template <int EPI, int NB, bool KCAT, int WF, bool SV, int NW, int QF, int NT>
__device__ __forceinline__ void stream_rows_tile(const GemmArgs& g, const TileCoord& tc,
                                                 char* xs) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    constexpr bool FP8 = WF == WF_FP8, FP4 = WF == WF_MXFP4, QW = WF != WF_BF16;
    constexpr int SRN = 16 * NW;
    constexpr int CS = (NB == 4 ? 8 : 16) * (NW / 8);  // k-steps (of 32) per token chunk
    constexpr int UNIT = FP4 ? 4 : FP8 ? 2 : 1;  // k-steps per weight load
    constexpr int PD = FP8 && NB == 4 ? 4 : 8;  // weight loads in flight
    constexpr int UPC = CS / UNIT;             // weight loads per chunk
    // chunks per loop iteration: the ring of PD loads turns a whole number
    // of times per iteration, so every slot index is static
    constexpr int RC = PD > UPC ? PD / UPC : 1;
    constexpr int TU = RC * UPC;               // weight loads per ring turn
    // 1 KB token loads per wave per chunk; with QF > 1, TL loads per chunk,
    // one each for waves 0 .. TL-1
    constexpr int XI = QF == 1 ? CS * NB / NW : 1;
    constexpr int TL = CS / QF, RB = 16 / QF;
    constexpr int CHUNK = CS * NB * 1024;      // bytes of one token chunk
    static_assert(!(QW && KCAT), "quantised weights are grouped products only");
    static_assert(QF == 1 || (NB == 1 && !KCAT && CS % QF == 0 && TL <= NW), "token packing");
    static_assert(2 * CHUNK <= sx_bytes<NW>() && CS % UNIT == 0 && TU % PD == 0 && XI % NB == 0,
                  "stream tiling");
    // NT > 1 (expert down products with fp16 rows and whole-line loads, K a
    // multiple of 1024 and N of SRS): NT column tiles in a row, each a whole
    // number of chunks and ring turns
    static_assert(NT == 1 || (SV && EPI == EPI_F16), "column tiles per workgroup");
    constexpr int SRS = SW ? SRN / 2 : SRN;  // weight rows from one column tile to the next
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int l16 = lane & 15, g4 = lane >> 4;

    // 32-bit byte offsets from wave-uniform bases; every operand of one group
    // fits in 4 GiB (checked on the host).  Row bytes: K * 2 (bf16), K (FP8),
    // K / 2 (MXFP4).
    const int64_t wrow_bytes = FP4 ? g.K / 2 : FP8 ? g.K : (int64_t)g.K * 2;
    const int64_t group_bytes = FP4 ? g.b_gstride / 2 : FP8 ? g.b_gstride : g.b_gstride * 2;
    const char* Bb = (const char*)g.B + tc.group * group_bytes;
    const char* B2b = (const char*)g.B2;
    const char* Ab = (const char*)g.A;
    const char* A2b = (const char*)g.A2;
    int wrow;
    if (SW) {
        const int c = min(tc.nt * (SRN / 2) + wave * 8 + (l16 & 7), g.N - 1);
        wrow = l16 < 8 ? c : g.N + c;
    } else {
        wrow = min(tc.nt * SRN + wave * 16 + l16, g.N - 1);
    }
    const uint32_t wo = (uint32_t)(wrow * wrow_bytes) + g4 * 16;
    // PL (SV: K a multiple of 512 for MXFP4, 128 for FP8, 64 for bf16): a
    // load pair covers 128 bytes of the wave's 16 rows (2 * UNIT k-steps) as
    // whole cache lines: the even unit of the pair rows 0-7, the odd one rows
    // 8-15, each row read by 8 lanes (lane l: row l % 8, bytes 16 * (l / 8)
    // ..).  wpo[p] is the offset of unit parity p less p * 64, so that unit u
    // sits at wpo[u & 1] + 64 u.
    static_assert(!(SV && KCAT), "load pairs: one K segment");
    constexpr bool PL = SV;
    // k-steps of a lane's contiguous 16 * W bytes of a row: a lane takes
    // elements 8 * W * g4 .. of each 32 * W-deep block, 8 per step
    constexpr int W = PL ? 2 * UNIT : UNIT;
    uint32_t wpo[2] = {0u, 0u};
    if constexpr (PL) {
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            const int x = p * 8 + (lane & 7);  // wave row
            int rr;
            if (SW) {
                const int c = min(tc.nt * (SRN / 2) + wave * 8 + (x & 7), g.N - 1);
                rr = x < 8 ? c : g.N + c;
            } else {
                rr = min(tc.nt * SRN + wave * 16 + x, g.N - 1);
            }
            wpo[p] = (uint32_t)(rr * wrow_bytes) + 16 * (lane >> 3) - (uint32_t)(p * 64);
        }
    }
    const uint32_t wo2 = KCAT ? (uint32_t)((int64_t)wrow * g.K2 * 2) + g4 * 16 : 0u;
    // MXFP4 block exponents of this row: K / 32 bytes, 4 per load unit
    const char* Sb = FP4 ? (const char*)g.b_scale + tc.group * g.b_scale_gstride +
                               (int64_t)wrow * (g.K / 32)
                         : nullptr;
    // token rows past the tile's end load its last row (never stored)
    uint32_t xo[NB], xo2[NB];
    if constexpr (QF == 1) {
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const int r = min(tc.row0 + tb * 16 + l16, tc.row1 - 1);
            xo[tb] = (uint32_t)(a_row_of(g, r) * g.lda * 2) +
                     g4 * (16 * W);
            xo2[tb] = KCAT ? (uint32_t)((int64_t)r * g.lda2 * 2) + g4 * 16 : 0u;
        }
    } else {
        const int r = min(tc.row0 + lane % RB, tc.row1 - 1);
        xo[0] = (uint32_t)(a_row_of(g, r) * g.lda * 2) +
                ((lane / RB) & 3) * (16 * W);
        xo2[0] = 0u;
    }

    const int ns1 = g.K / 32;
    const int ns = ns1 + (KCAT ? g.K2 / 32 : 0);
    const int nch = (ns + CS - 1) / CS;
    const int nu = ns / UNIT;  // weight load units
    // MXFP4 block exponents, one dword per load unit.  K a multiple of 512:
    // they come in groups of 8 units (32 bytes of each row), one ring turn
    // and one loop pass, lane (row i, q) holding units 2 q and 2 q + 1 of
    // the group: one 8-byte load per wave for 8 units rather than a 16-byte
    // one for each chunk's 4, since the count of memory instructions and of
    // cache lines, not bytes, is what holds this stream back.  The group in
    // use (egc) is handed to the lanes that need it with ds_bpermute when a
    // chunk starts (bsc: the chunk's block scales for this lane); the next
    // one (egn) is requested when a pass starts, as far ahead as the
    // weights.  Otherwise (sxn, sxc) a chunk's exponent dwords travel with
    // its token rows, one chunk ahead, byte g4 of dword j for this lane.
    typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
    uint32_t sxn[FP4 && !SV ? UPC : 1], sxc[FP4 && !SV ? UPC : 1];
    u32x2_t egc = u32x2_t{0u, 0u}, egn = egc;
    float bsc[FP4 && SV ? UPC : 1];
    // NT > 1: unit u of the workgroup's stream is unit u - t * nu of column
    // tile t, whose rows lie SRS * t rows on; since a row is nu units of 64
    // bytes, its address is the tile-0 address of unit u shifted by
    // t * (SRS - 1) rows.  Exponent rows move SRS * K / 32 bytes per tile.
    const uint32_t tstep = NT > 1 ? (uint32_t)((SRS - 1) * wrow_bytes) : 0u;
    const uint32_t xstep = NT > 1 ? (uint32_t)(SRS * (g.K / 32)) : 0u;

    // Token chunk c lives in LDS buffer c & 1 as 1 KB blocks b = (k-step
    // b / NB, 16-row block b % NB), each in MFMA operand order (lane l holds
    // row l % 16 and the 8 k of the step that lane l / 16 takes).  This wave
    // moves blocks wave * XI .. +XI-1; steps past K re-read the last step
    // (never used).
    u32x4_t xr[XI];
    // byte offset of step st's 8 elements for a lane (the k order of the
    // weight loads; the lane's g4 part is in xo)
    auto step_off = [&](int st) __attribute__((always_inline)) {
        return (uint32_t)(st / W) * (64 * W) + (uint32_t)(st % W) * 16;
    };
    // chunk c of column tile xt (tokens do not depend on the tile)
    auto load_x = [&](int c, int xt) __attribute__((always_inline)) {
        if constexpr (QF > 1) {
            if (wave < TL) {
                const int st = min(c * CS + wave * QF + lane / (4 * RB), ns - 1);
                xr[0] = *(const u32x4_t*)(Ab + (xo[0] + step_off(st)));
            }
        } else {
#pragma unroll
            for (int i = 0; i < XI; ++i) {
                const int b = wave * XI + i;
                const int tb = i % NB;
                const int st = min(c * CS + b / NB, ns - 1);
                const bool seg1 = !KCAT || st < ns1;
                const char* src = seg1 ? Ab + (xo[tb] + step_off(st))
                                       : A2b + (xo2[tb] + (uint32_t)(st - ns1) * 64);
                xr[i] = *(const u32x4_t*)src;
            }
        }
        // MXFP4, K not a multiple of 512: the chunk's exponent dwords
        if constexpr (FP4 && !SV) {
#pragma unroll
            for (int j = 0; j < UPC; ++j)
                sxn[j] = *(const uint32_t*)(Sb + 4 * min(c * UPC + j, nu - 1));
        }
    };
    // MXFP4, K a multiple of 512: exponent group gi of column tile xt into
    // egn (units past the row's end re-read its last 2)
    auto load_eg = [&](int gi, int xt) __attribute__((always_inline)) {
        if constexpr (FP4 && SV) {
            static_assert(UPC * RC == 8 && PD == 8, "one exponent group per pass");
            const int u0 = min(8 * gi + 2 * g4, nu - 2);
            egn = *(const u32x2_t*)(Sb + (NT > 1 ? xt * xstep : 0u) + 4 * u0);
        }
    };
    // into LDS buffer c & 1; cl is the chunk's place in its column tile
    auto store_x = [&](int c, int cl) __attribute__((always_inline)) {
        if constexpr (QF > 1) {
            if (wave < TL) {
                const int sl = wave * QF + lane / (4 * RB);  // step within the chunk
                const int p = lane % RB + 16 * ((lane / RB) & 3);  // its operand lane
                if (QW && cl * CS + sl >= ns) xr[0] = u32x4_t{0u, 0u, 0u, 0u};
                *(u32x4_t*)(xs + (c & 1) * CHUNK + sl * 1024 + p * 16) = xr[0];
            }
        } else {
            char* dst = xs + (c & 1) * CHUNK + lane * 16;
#pragma unroll
            for (int i = 0; i < XI; ++i) {
                // FP8 / MXFP4: steps past K get zero tokens (once per chunk,
                // in place of a select per step on the converted weights)
                if (QW && cl * CS + (wave * XI + i) / NB >= ns)
                    xr[i] = u32x4_t{0u, 0u, 0u, 0u};
                *(u32x4_t*)(dst + (wave * XI + i) * 1024) = xr[i];
            }
        }
        if constexpr (FP4 && !SV) {
#pragma unroll
            for (int j = 0; j < UPC; ++j) sxc[j] = sxn[j];
        }
    };
    // NT > 1: loads run at most PD <= nu units ahead, so unit u lies in the
    // tile of the MFMAs (shift wsh) or the next one (from unit wu_end on)
    int wu_end = nu;
    uint32_t wsh = 0u, wsh_next = tstep;
    // Weight load unit u covers k-steps UNIT*u .. +UNIT-1, 64 bytes of the
    // row.  Whole-line (PL) weight loads are non-temporal: each weight line
    // is read once, and L2 keeps the token rows that the workgroups of an
    // expert's column tiles share (MXFP4 gate/up: HBM fetch 1.08x -> 1.03x
    // of its algorithmic bytes).  Half-line loads (the second K segment,
    // unaligned K) stay ordinary: the two halves of a line come from two
    // instructions, and non-temporal reads of them ran 22% slower.
    auto load_w = [&](int u) __attribute__((always_inline)) {
        if constexpr (NT > 1) {
            u = min(u, NT * nu - 1);
            const uint32_t sh = u >= wu_end ? wsh_next : wsh;
            return __builtin_nontemporal_load(
                (const u32x4_t*)(Bb + (wpo[u & 1] + sh + (uint32_t)u * 64)));
        }
        u = min(u, nu - 1);
        if constexpr (PL)
            return __builtin_nontemporal_load((const u32x4_t*)(Bb + (wpo[u & 1] + (uint32_t)u * 64)));
        const bool seg1 = !KCAT || u < ns1;
        const char* src = seg1 ? Bb + (wo + (uint32_t)u * 64)
                               : B2b + (wo2 + (uint32_t)(u - ns1) * 64);
        return *(const u32x4_t*)src;
    };

    // MXFP4 single-block tiles alternate two accumulators so that
    // consecutive MFMAs do not wait on each other
    constexpr int NACC = FP4 && NB == 1 ? 2 : 1;
    f32x4_t acc[NB], acc2[NB];
#pragma unroll
    for (int tb = 0; tb < NB; ++tb) acc[tb] = acc2[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    u32x4_t w[PD];

    // The first weight fragments go out before the wait for chunk 0.  Order
    // is pinned (empty asm with a memory clobber) so that on both paths into
    // the store of chunk c + 1 the token loads are followed by exactly the
    // weight loads of chunk c: the compiler's wait for the token registers
    // then leaves the newest weight loads in flight.
    load_x(0, 0);
    load_eg(0, 0);
    asm volatile("" ::: "memory");
#pragma unroll
    for (int v = 0; v < PD; ++v) w[v] = load_w(v);
    asm volatile("" ::: "memory");
    store_x(0, 0);
    asm volatile("" ::: "memory");
    load_x(1, 0);  // NT > 1 has nch >= 2
    asm volatile("" ::: "memory");
    // NT > 1: the place in its tile of the chunk loaded but not stored, and
    // the place xl2 in tile xt2 of the next chunk to load
    int xs1 = 1, xl2 = 2, xt2 = 0;
    if (NT > 1 && xl2 == nch) xl2 = 0, xt2 = 1;

    // Chunk c starts once this wave's LDS writes of chunk c are done, and
    // its LDS reads of chunk c - 1; after the barrier every wave's part of
    // chunk c is visible and no wave reads buffer (c + 1) & 1 any more.  (A
    // __syncthreads fence would also drain the weight loads in flight.)
    auto chunk_begin = [&](int c) __attribute__((always_inline)) {
        wait_lgkm0();
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        return (const char*)(xs + (c & 1) * CHUNK + lane * 16);
    };
    // Load unit j of chunk c, held in ring slot v: its UNIT k-steps against
    // every token block, then the refill of the slot PD units ahead.
    // A load pair (slots va = v - 1 and v) is used with its odd unit: lanes
    // l and l ^ 8 hold the two halves of the lines of row l % 8 (even unit)
    // and of row 8 + l % 8 (odd unit); one row-rotate by 8 and three selects
    // per dword give lane l (row l % 16) bytes 32 q .. +15 (q = l / 16) of
    // the row's 128 in a and the next 16 in b.
    struct Pair {
        u32x4_t a, b;
    };
    auto exchange = [&](int va, int v) __attribute__((always_inline)) {
        const bool lo = (lane & 8) == 0;
        Pair p;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const uint32_t sv = lo ? w[v][d] : w[va][d];
            const uint32_t t = (uint32_t)__builtin_amdgcn_update_dpp(
                0, (int)sv, 0x128 /* row_ror:8 */, 0xf, 0xf, false);
            p.a[d] = lo ? w[va][d] : t;
            p.b[d] = lo ? t : w[v][d];
        }
        return p;
    };
    auto unit = [&](int c, const char* xc, int j, int v) __attribute__((always_inline)) {
        if constexpr (PL) {
            if (j & 1) {
                const int va = v - 1, ja = j - 1;
                const Pair p = exchange(va, v);
                w[va] = load_w(c * UPC + ja + PD);
                w[v] = load_w(c * UPC + j + PD);
                asm volatile("" ::: "memory");
                if constexpr (FP4) {
                    // 32 codes in a, 32 in b; step h of the 8 takes codes
                    // 8 h .. of the 64, with the block scale of a or b
                    constexpr int XG = 4 / NB;
#pragma unroll
                    for (int h0 = 0; h0 < 2 * UNIT; h0 += XG) {
                        u32x4_t xv[XG][NB];
#pragma unroll
                        for (int hh = 0; hh < XG; ++hh)
#pragma unroll
                            for (int tb = 0; tb < NB; ++tb)
                                xv[hh][tb] = *(const u32x4_t*)(xc + ((ja * UNIT + h0 + hh) * NB + tb) *
                                                                       1024);
#pragma unroll
                        for (int hh = 0; hh < XG; ++hh) {
                            const int h = h0 + hh;
                            const bf16x8_t wf = __builtin_bit_cast(
                                bf16x8_t, fp4x8_to_bf16x8(h < 4 ? p.a[h] : p.b[h - 4],
                                                          bsc[ja + (h >= 4)]));
#pragma unroll
                            for (int tb = 0; tb < NB; ++tb) {
                                f32x4_t& a = NACC == 2 && (hh & 1) ? acc2[tb] : acc[tb];
                                a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                    wf, __builtin_bit_cast(bf16x8_t, xv[hh][tb]), a, 0, 0, 0);
                            }
                        }
                    }
                } else {
                    // FP8: 16 codes in a, 16 in b, step h of the 4 takes codes
                    // 8 h ..; bf16: step 0 takes a, step 1 b (steps past K,
                    // the ragged last chunk, multiply zero weights)
#pragma unroll
                    for (int h = 0; h < 2 * UNIT; ++h) {
                        const int sl = ja * UNIT + h;  // step within the chunk
                        u32x4_t wf;
                        if constexpr (FP8) {
                            const u32x4_t& q = h < 2 ? p.a : p.b;
                            wf = fp8x8_to_bf16x8(q[2 * (h & 1)], q[2 * (h & 1) + 1]);
                        } else {
                            // steps past K (a ragged last chunk) multiply zero
                            // weights; with NT > 1, c counts the chunks of all
                            // tiles, and K (a multiple of 1024) leaves none ragged
                            wf = NT > 1 || c * CS + sl < ns ? (h == 0 ? p.a : p.b)
                                                            : u32x4_t{0u, 0u, 0u, 0u};
                        }
#pragma unroll
                        for (int tb = 0; tb < NB; ++tb) {
                            const u32x4_t xv = *(const u32x4_t*)(xc + (sl * NB + tb) * 1024);
                            acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, wf), __builtin_bit_cast(bf16x8_t, xv),
                                acc[tb], 0, 0, 0);
                        }
                    }
                }
            }
            return;
        }
        if constexpr (FP4) {
            // token fragments 4 at a time (XG steps of NB blocks) ahead of
            // their MFMAs, so their LDS latency overlaps; zero tokens
            // already cover steps past K
            constexpr int XG = 4 / NB;
            const float bs = e8m0_scale((sxc[j] >> (8 * g4)) & 0xffu);
#pragma unroll
            for (int h0 = 0; h0 < UNIT; h0 += XG) {
                u32x4_t xv[XG][NB];
#pragma unroll
                for (int hh = 0; hh < XG; ++hh)
#pragma unroll
                    for (int tb = 0; tb < NB; ++tb)
                        xv[hh][tb] =
                            *(const u32x4_t*)(xc + ((j * UNIT + h0 + hh) * NB + tb) * 1024);
#pragma unroll
                for (int hh = 0; hh < XG; ++hh) {
                    const bf16x8_t wf =
                        __builtin_bit_cast(bf16x8_t, fp4x8_to_bf16x8(w[v][h0 + hh], bs));
#pragma unroll
                    for (int tb = 0; tb < NB; ++tb) {
                        f32x4_t& a = NACC == 2 && (hh & 1) ? acc2[tb] : acc[tb];
                        a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            wf, __builtin_bit_cast(bf16x8_t, xv[hh][tb]), a, 0, 0, 0);
                    }
                }
            }
            w[v] = load_w(c * UPC + j + PD);
            asm volatile("" ::: "memory");
            return;
        }
#pragma unroll
        for (int hh = 0; hh < UNIT; ++hh) {
            const int sl = j * UNIT + hh;  // step within the chunk
            const int st = c * CS + sl;
            u32x4_t wv = w[v];
            if (FP8) wv = fp8x8_to_bf16x8(w[v][2 * hh], w[v][2 * hh + 1]);
            // bf16: steps past K (the ragged last chunk) multiply zero weights
            const u32x4_t wz = FP8 || st < ns ? wv : u32x4_t{0u, 0u, 0u, 0u};
            const bf16x8_t wf = __builtin_bit_cast(bf16x8_t, wz);
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) {
                const u32x4_t xv = *(const u32x4_t*)(xc + (sl * NB + tb) * 1024);
                acc[tb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    wf, __builtin_bit_cast(bf16x8_t, xv), acc[tb], 0, 0, 0);
            }
        }
        const int ul = c * UPC + j;
        w[v] = load_w(ul + PD);
        // keep each refill where its slot frees up (the scheduler otherwise
        // sinks them all to the end of the chunk)
        if (QW) asm volatile("" ::: "memory");
    };
    // chunk c + 1 has had a whole chunk to arrive; chunks past the end only
    // touch the idle buffer, which keeps this branch-free
    auto chunk_end = [&](int c) __attribute__((always_inline)) {
        asm volatile("" ::: "memory");
        store_x(c + 1, NT > 1 ? xs1 : c + 1);
        asm volatile("" ::: "memory");
        if constexpr (NT > 1) {
            // past the last tile: in-bounds re-reads into the idle buffer
            load_x(xl2, xt2);
            xs1 = xl2;
            if (++xl2 == nch) xl2 = 0, xt2 = min(xt2 + 1, NT - 1);
        } else {
            load_x(c + 2, 0);
        }
        asm volatile("" ::: "memory");
    };

    // Stores column tile nt of the output from acc (+ acc2).
    auto epilogue = [&](int nt) __attribute__((always_inline)) {
        if constexpr (NACC == 2) {
#pragma unroll
            for (int tb = 0; tb < NB; ++tb) acc[tb] += acc2[tb];
        }

        // row scales of FP8 weights, for the 4 weight rows this lane's sums belong to
        float rs[4] = {1.f, 1.f, 1.f, 1.f};
        if (FP8) {
            const float* sc = (const float*)g.b_scale + (int64_t)tc.group * g.b_scale_gstride;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                int n;
                if (SW) {
                    const int hc = min(nt * (SRN / 2) + wave * 8 + (g4 & 1) * 4 + j, g.N - 1);
                    n = g4 < 2 ? hc : g.N + hc;
                } else {
                    n = min(nt * SRN + wave * 16 + g4 * 4 + j, g.N - 1);
                }
                rs[j] = sc[n];
            }
        }

        // acc[tb][j] = C[weight row 4*g4 + j of this wave][token 16*tb + l16]
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) {
            const int r = tc.row0 + tb * 16 + l16;
            if (SW) {
                // lanes 32..63 hold the up rows of lane - 32's gate rows
                float up[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) up[j] = __shfl_xor(acc[tb][j] * rs[j], 32);
                if (g4 < 2 && r < tc.row1) {
                    bf16_t* crow = (bf16_t*)g.C + (int64_t)r * g.ldc;
                    const int hc0 = nt * (SRN / 2) + wave * 8 + g4 * 4;
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        if (hc0 + j < g.N)
                            crow[hc0 + j] = f32_to_bf16(glu_f32(acc[tb][j] * rs[j], up[j], g));
                }
            } else if (EPI == EPI_F16) {
                // four consecutive fp16 columns in one 8-byte store (N and the
                // column base are multiples of 4, so they are all in range or none)
                const int c0 = nt * SRN + wave * 16 + g4 * 4;
                if (r < tc.row1 && c0 < g.N)
                    *(uint2*)((uint16_t*)g.C + (int64_t)r * g.ldc + c0) =
                        make_uint2(pack_f16x2(acc[tb][0] * rs[0], acc[tb][1] * rs[1]),
                                   pack_f16x2(acc[tb][2] * rs[2], acc[tb][3] * rs[3]));
            } else if (r < tc.row1) {
                const int c0 = nt * SRN + wave * 16 + g4 * 4;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int c = c0 + j;
                    if (c >= g.N) continue;
                    float o = acc[tb][j] * rs[j];
                    if (EPI == EPI_F32_BIAS && g.bias) o += g.bias[c];
                    if (EPI == EPI_OUT)
                        ((bf16_t*)g.C)[(int64_t)r * g.ldc + c] = f32_to_bf16(o);
                    else
                        ((float*)g.C)[(int64_t)r * g.ldc + c] = o;
                }
            }
        }
    };

    // NT > 1: after a tile's last chunk its sums are stored and cleared
    // while the loads of the next tile are in flight
    auto next_tile = [&](int& tile) __attribute__((always_inline)) {
        epilogue(tc.nt + tile);
#pragma unroll
        for (int tb = 0; tb < NB; ++tb) acc[tb] = acc2[tb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        ++tile;
        wsh = wsh_next;
        wsh_next += tstep;
        wu_end += nu;
    };
    if constexpr (RC == 1) {
        // one chunk turns the ring of PD loads a whole number of times
        int tile = 0, tleft = nch;
        for (int c = 0; c < NT * nch; ++c) {
            const char* xc = chunk_begin(c);
#pragma unroll
            for (int u = 0; u < UPC; u += PD)
#pragma unroll
                for (int v = 0; v < PD; ++v) unit(c, xc, u + v, v);
            chunk_end(c);
            if constexpr (NT > 1) {
                if (--tleft == 0 && tile < NT - 1) {
                    next_tile(tile);
                    tleft = nch;
                }
            }
        }
        epilogue(tc.nt + tile);
        return;
    } else {
        // MXFP4: a chunk holds fewer than PD loads; RC chunks turn the ring
        // once (unit c * UPC + j of chunk c = c0 + r sits in slot r * UPC + j).
        // Chunks past the end (when RC does not divide nch) multiply zero
        // weights and stage clamped, in-bounds token steps.
        // NT > 1: when a tile's last chunk is done, its sums are stored
        // and cleared while the loads of the next tile are in flight
        int tile = 0, tleft = nch;
        for (int c0 = 0; c0 < NT * nch; c0 += RC) {
            if constexpr (FP4 && SV) {
                // this pass's exponent group comes into use; the next pass's
                // (the next group of the tile, or the next tile's first)
                egc = egn;
                if (NT > 1 && tleft == RC) load_eg(0, min(tile + 1, NT - 1));
                else load_eg((NT > 1 ? nch - tleft : c0) / RC + 1, tile);
                asm volatile("" ::: "memory");
            }
#pragma unroll
            for (int r = 0; r < RC; ++r) {
                const int c = c0 + r;
                const char* xc = chunk_begin(c);
                if constexpr (FP4 && SV) {
                    // pair pp of the chunk, units 2 pp and 2 pp + 1 of it
                    // (blocks 0-3 and 4-7 of its 128 bytes per row), is pair
                    // k = r * UPC / 2 + pp of the group, held by lane (i, k);
                    // this lane's codes a and b are blocks 2 q and 2 q + 1
#pragma unroll
                    for (int pp = 0; pp < UPC / 2; ++pp) {
                        const int src = (l16 + 16 * (r * UPC / 2 + pp)) * 4;
                        const uint32_t d0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)egc[0]);
                        const uint32_t d1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)egc[1]);
                        const uint32_t d = g4 < 2 ? d0 : d1;
                        const uint32_t sh = 16 * (g4 & 1);
                        bsc[2 * pp] = e8m0_scale((d >> sh) & 0xffu);
                        bsc[2 * pp + 1] = e8m0_scale((d >> (sh + 8)) & 0xffu);
                    }
                    asm volatile("" ::: "memory");
                }
#pragma unroll
                for (int j = 0; j < UPC; ++j) unit(c, xc, j, r * UPC + j);
                chunk_end(c);
            }
            if constexpr (NT > 1) {
                tleft -= RC;
                if (tleft == 0 && tile < NT - 1) {
                    next_tile(tile);
                    tleft = nch;
                }
            }
        }
        epilogue(tc.nt + tile);
    }
}

// Grouped tiles here hold one whole group of at most 64 rows; dense products
// are cut into 16-row tiles.
// SV (MXFP4 with K a multiple of 512): whole-line weight loads and exponent
// groups.
// NT: column tiles per workgroup, streamed back to back (ntn a multiple of NT).
template <int EPI, bool KCAT, int WF, bool SV, int NW, int NT>
__global__ __launch_bounds__(64 * NW, 4) void gemm_bf16_stream(GemmArgs g) {
    constexpr bool SW = EPI == EPI_SWIGLU;
    constexpr int SRN = 16 * NW;
    const int ntn = SW ? (g.N + SRN / 2 - 1) / (SRN / 2) : (g.N + SRN - 1) / SRN;
    TileCoord tc;
    if (!fetch_tile(g, SROWS, ntn / NT, tc)) return;
    tc.nt *= NT;
    __shared__ __attribute__((aligned(1024))) char xs[sx_bytes<NW>()];
    const int rows = tc.row1 - tc.row0;
    // (not with FP8 weights, whose register budget the packed forms push
    // into spills inside the 2-block loop)
    if constexpr (!KCAT && WF != WF_FP8) {
        if (rows <= 4) {
            stream_rows_tile<EPI, 1, KCAT, WF, SV, NW, 4, NT>(g, tc, xs);
            return;
        }
        if (rows <= 8) {
            stream_rows_tile<EPI, 1, KCAT, WF, SV, NW, 2, NT>(g, tc, xs);
            return;
        }
    }
    if (rows <= 16) stream_rows_tile<EPI, 1, KCAT, WF, SV, NW, 1, NT>(g, tc, xs);
    else if (rows <= 32) stream_rows_tile<EPI, 2, KCAT, WF, SV, NW, 1, NT>(g, tc, xs);
    else stream_rows_tile<EPI, 4, KCAT, WF, SV, NW, 1, NT>(g, tc, xs);
}

// Dense products with fewer workgroups than this split K over the waves.
constexpr int64_t kStreamRowsMinGrid = 1024;

template <bool KC, int WF, bool SV, int NW, int NT = 1>
void launch_stream_rows(const GemmArgs& g, int nm, hipStream_t s) {
    const dim3 gd((unsigned)((int64_t)nm * (stream_col_tiles_nw(g.epi, g.N, NW) / NT))),
        bd(64 * NW);
    if constexpr (NT > 1) {
        // only the expert down product's fp16 rows take several tiles
        if (g.epi == EPI_F16) gemm_bf16_stream<EPI_F16, KC, WF, SV, NW, NT><<<gd, bd, 0, s>>>(g);
    } else {
        switch (g.epi) {
            case EPI_F16:
                // grouped expert rows only (never a K-concatenated product)
                if constexpr (!KC) gemm_bf16_stream<EPI_F16, KC, WF, SV, NW, NT><<<gd, bd, 0, s>>>(g);
                break;
            case EPI_F32: gemm_bf16_stream<EPI_F32, KC, WF, SV, NW, NT><<<gd, bd, 0, s>>>(g); break;
            case EPI_F32_BIAS:
                gemm_bf16_stream<EPI_F32_BIAS, KC, WF, SV, NW, NT><<<gd, bd, 0, s>>>(g);
                break;
            case EPI_OUT: gemm_bf16_stream<EPI_OUT, KC, WF, SV, NW, NT><<<gd, bd, 0, s>>>(g); break;
            default: gemm_bf16_stream<EPI_SWIGLU, KC, WF, SV, NW, NT><<<gd, bd, 0, s>>>(g); break;
        }
    }
}

// Column tiles per workgroup of a quantised expert down product (fp16 rows)
// with whole-line weight loads: with short rows (K = 2048 is 16 MXFP4 or 32
// FP8 load units per row) one tile's stream is mostly the filling and
// draining of the loads in flight, so a workgroup streams several tiles back
// to back, each a whole number of chunks and ring turns (K a multiple of
// 1024) of whole tiles (N a multiple of 128).  Decode down product with
// paired runs: FP8 0.850-0.853 -> 0.819-0.820 ms; bf16 rows (64 units at
// K = 2048) 1.55-1.58 -> 1.62 ms, so bf16 keeps one tile.  Gate/up rows
// (K = 7168) gain nothing from it.
int stream_tiles_per_group(const GemmArgs& g) {
    if (g.epi != EPI_F16 || g.K % 1024 != 0 || g.N % 128 != 0) return 1;
    const int ntn = g.N / 128;
    // 2 tiles (32 units per row at K = 2048) measured faster than 4 or 1
    return g.K <= 4096 && ntn % 2 == 0 ? 2 : 1;
}

}  // namespace

int stream_row_tile() { return SROWS; }

int stream_col_tiles(int epi, int N) { return stream_col_tiles_nw(epi, N, 8); }

hipError_t launch_stream_gemm(const GemmArgs& g, int nm, hipStream_t s) {
    const bool sw = g.epi == EPI_SWIGLU;
    const int64_t grid_ks = (int64_t)nm * (sw ? (g.N + 31) / 32 : (g.N + SNW - 1) / SNW);
    if (grid_ks <= 0) return hipSuccess;
    if (g.epi == EPI_F16 && (!g.tiles || g.A2)) return hipErrorInvalidValue;
    if (!g.tiles && grid_ks < kStreamRowsMinGrid && g.b_fmt == WF_BF16) {
        const dim3 gd((unsigned)grid_ks), bd(256);
        switch (g.epi) {
            case EPI_F32: gemm_bf16_stream_ksplit<EPI_F32><<<gd, bd, 0, s>>>(g); break;
            case EPI_F32_BIAS: gemm_bf16_stream_ksplit<EPI_F32_BIAS><<<gd, bd, 0, s>>>(g); break;
            case EPI_OUT: gemm_bf16_stream_ksplit<EPI_OUT><<<gd, bd, 0, s>>>(g); break;
            default: gemm_bf16_stream_ksplit<EPI_SWIGLU><<<gd, bd, 0, s>>>(g); break;
        }
    } else {
        if (g.b_fmt != WF_BF16 && g.A2) return hipErrorInvalidValue;
        if (g.b_fmt == WF_MXFP4 && g.K % 128 != 0) return hipErrorInvalidValue;
        if (g.b_fmt == WF_FP8 && g.K % 128 == 0) {
            if (stream_tiles_per_group(g) == 2)
                launch_stream_rows<false, WF_FP8, true, 8, 2>(g, nm, s);
            else
                launch_stream_rows<false, WF_FP8, true, 8>(g, nm, s);
        } else if (g.b_fmt == WF_FP8) {
            launch_stream_rows<false, WF_FP8, false, 8>(g, nm, s);
        } else if (g.b_fmt == WF_MXFP4 && g.K % 512 == 0) {
            if (stream_tiles_per_group(g) == 2)
                launch_stream_rows<false, WF_MXFP4, true, 8, 2>(g, nm, s);
            else
                launch_stream_rows<false, WF_MXFP4, true, 8>(g, nm, s);
        } else if (g.b_fmt == WF_MXFP4) {
            launch_stream_rows<false, WF_MXFP4, false, 8>(g, nm, s);
        } else if (g.A2) {
            launch_stream_rows<true, WF_BF16, false, 8>(g, nm, s);
        } else if (g.K % 64 == 0) {
            launch_stream_rows<false, WF_BF16, true, 8>(g, nm, s);
        } else {
            launch_stream_rows<false, WF_BF16, false, 8>(g, nm, s);
        }
    }
    return hipGetLastError();
}

}  // namespace moe
