// gemm.hip -- block-scaled INT8 GEMM on the gfx950 INT8 matrix cores.
//
// Pages: Jetfire summary, "Approach": linear operators (forward, activation
// gradient and weight gradient) consume INT8 codes with one scale per 32x32
// block and produce INT8 + per-block scales, quantized on-chip.
//
//   C[M x N] = op(A)[M x K] . op(B)[K x N]
//   per output block (I, J), per 32-deep k-block kappa (ascending):
//     P     = exact int32 sum of 32 code products   (one MFMA)
//     sigma = fl(sA[I,kappa] * sB[kappa,J])
//     acc   = fma(sigma, (float)P, acc)              (binary32, VALU)
//   epilogue: store acc (fp32) or requantize the 32x32 block in registers.
//
// One v_mfma_i32_32x32x32_i8 is exactly one (32x32 output block, k-block)
// pair: its K of 32 matches the scale block, so every MFMA result is the
// exact int32 partial that gets rescaled.  The operands are passed to the
// MFMA swapped (B fragment first) so that a lane owns one output ROW and
// its 16 accumulators are columns 8g + 4h + r (g, r = 0..3, h = lane/32):
// that layout gives 4-column (16-byte fp32 / 4-byte int8) stores and keeps
// a block's requantization inside one wavefront.
//
// Operand staging.  Both operands are staged through LDS as [row][k] byte
// tiles (k contiguous), whatever their storage order:
//   k-contiguous storage (A with transA=0, B with transB=1): 16-byte global
//     loads copied to LDS as they are;
//   row-contiguous storage (A with transA=1, B with transB=0): each thread
//     loads a 4(k) x 4(row) byte square with four dword loads and transposes
//     it in registers (byte permutes) before writing four dwords to LDS.
// A 32x32 block is square, so the transposed operand of the gradients keeps
// its codes and its scale; only the scale-grid index order changes.
//
// Workgroup: 4 wavefronts as 2 x 2; wavefront tile WM x WN output blocks;
// LDS double-buffered over stages of KB k-blocks.
#include "jf_device.h"
#include "jf_launch.h"

namespace jf {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kThreads = 256;
constexpr int kPad = 16;  // bytes of padding per LDS row

// Transpose a 4x4 byte square: in[t] holds 4 consecutive row-bytes of k-row t;
// out[r] holds the 4 k-bytes of row r (k ascending from the low byte).
__device__ __forceinline__ void transpose4x4(const uint32_t in[4], uint32_t out[4]) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
        out[r] = ((in[0] >> (8 * r)) & 0xffu) | (((in[1] >> (8 * r)) & 0xffu) << 8) |
                 (((in[2] >> (8 * r)) & 0xffu) << 16) | (((in[3] >> (8 * r)) & 0xffu) << 24);
}

// One operand tile: R logical rows (output rows for A, output columns for B)
// by BK k-bytes, staged global -> registers -> LDS.
template <int R, int BK, bool KC>
struct Tile {
    static constexpr int P = BK + kPad;                       // LDS row pitch (bytes)
    static constexpr int kPieces = R * BK / 16;               // 16-byte pieces per stage
    static constexpr int kPer = kPieces / kThreads;
    static_assert(kPieces % kThreads == 0, "tile must split evenly over the workgroup");
    uint32_t reg[kPer][4];

    // base: operand base pointer; ld: stored leading dimension; row0: first
    // logical row of the tile; nrows: logical rows of the operand (a
    // multiple of 32); k0: first k of the stage; K: total k.
    __device__ __forceinline__ void load(const int8_t *__restrict__ base, int64_t ld, int row0, int nrows,
                                         int k0, int K, int tid) {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const int c = tid + kThreads * p;
            if constexpr (KC) {
                const int r = c / (BK / 16), kc = c % (BK / 16);
                const int grow = min(row0 + r, nrows - 1);
                const int k = k0 + 16 * kc;
                if (k < K) {
                    const uint4 v = *reinterpret_cast<const uint4 *>(base + (int64_t)grow * ld + k);
                    reg[p][0] = v.x; reg[p][1] = v.y; reg[p][2] = v.z; reg[p][3] = v.w;
                } else {
                    reg[p][0] = reg[p][1] = reg[p][2] = reg[p][3] = 0u;
                }
            } else {
                const int kg = c / (R / 4), rg = c % (R / 4);
                const int gcol = min(row0 + 4 * rg, nrows - 4);
                const int k = k0 + 4 * kg;
                uint32_t in[4];
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    in[t] = (k < K) ? *reinterpret_cast<const uint32_t *>(base + (int64_t)(k + t) * ld + gcol) : 0u;
                transpose4x4(in, reg[p]);
            }
        }
    }

    __device__ __forceinline__ void store(int8_t *__restrict__ lds, int tid) const {
#pragma unroll
        for (int p = 0; p < kPer; ++p) {
            const int c = tid + kThreads * p;
            if constexpr (KC) {
                const int r = c / (BK / 16), kc = c % (BK / 16);
                *reinterpret_cast<uint4 *>(lds + r * P + 16 * kc) =
                    make_uint4(reg[p][0], reg[p][1], reg[p][2], reg[p][3]);
            } else {
                const int kg = c / (R / 4), rg = c % (R / 4);
#pragma unroll
                for (int t = 0; t < 4; ++t) *reinterpret_cast<uint32_t *>(lds + (4 * rg + t) * P + 4 * kg) = reg[p][t];
            }
        }
    }
};

template <int WM, int WN, int KB, bool A_KC, bool B_KC, bool OUT_I8>
__global__ __launch_bounds__(kThreads) void k_gemm_i8bs(
    const int8_t *__restrict__ A, int64_t lda, const float *__restrict__ sA, int64_t ldsa,
    const int8_t *__restrict__ B, int64_t ldb, const float *__restrict__ sB, int64_t ldsb,
    int M, int N, int K, void *__restrict__ Cv, int64_t ldc, float *__restrict__ sC, int tilesN) {
    constexpr int BM = 2 * WM * kBlock, BN = 2 * WN * kBlock, BK = KB * kBlock;
    using TA = Tile<BM, BK, A_KC>;
    using TB = Tile<BN, BK, B_KC>;
    __shared__ __attribute__((aligned(16))) int8_t lds_a[2][BM * TA::P];
    __shared__ __attribute__((aligned(16))) int8_t lds_b[2][BN * TB::P];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wave = wave_id_uniform();
    const int wr = wave >> 1, wc = wave & 1;

    const int tm = blockIdx.x / tilesN, tn = blockIdx.x - tm * tilesN;
    const int row0 = tm * BM, col0 = tn * BN;
    const int nbM = M / kBlock, nbN = N / kBlock, nkb = K / kBlock;
    const int I0 = row0 / kBlock + wr * WM, J0 = col0 / kBlock + wc * WN;

    float acc[WM][WN][16];
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;

    const int nstage = (nkb + KB - 1) / KB;
    TA ta;
    TB tb;
    if (nstage > 0) {
        ta.load(A, lda, row0, M, 0, K, tid);
        tb.load(B, ldb, col0, N, 0, K, tid);
        ta.store(lds_a[0], tid);
        tb.store(lds_b[0], tid);
    }
    __syncthreads();

    const int frag_row = lane & 31, frag_k = 16 * (lane >> 5);
    const v16i zero = {};

    for (int st = 0; st < nstage; ++st) {
        const int buf = st & 1;
        const bool more = st + 1 < nstage;
        if (more) {
            ta.load(A, lda, row0, M, (st + 1) * BK, K, tid);
            tb.load(B, ldb, col0, N, (st + 1) * BK, K, tid);
        }
#pragma unroll
        for (int kk = 0; kk < KB; ++kk) {
            const int kb = st * KB + kk;
            if (kb >= nkb) break;
            v4i af[WM], bf[WN];
            float sa[WM], sb[WN];
#pragma unroll
            for (int a = 0; a < WM; ++a) {
                af[a] = *reinterpret_cast<const v4i *>(lds_a[buf] + ((wr * WM + a) * kBlock + frag_row) * TA::P +
                                                       kk * kBlock + frag_k);
                const int I = min(I0 + a, nbM - 1);
                sa[a] = A_KC ? sA[(int64_t)I * ldsa + kb] : sA[(int64_t)kb * ldsa + I];
            }
#pragma unroll
            for (int b = 0; b < WN; ++b) {
                bf[b] = *reinterpret_cast<const v4i *>(lds_b[buf] + ((wc * WN + b) * kBlock + frag_row) * TB::P +
                                                       kk * kBlock + frag_k);
                const int J = min(J0 + b, nbN - 1);
                sb[b] = B_KC ? sB[(int64_t)J * ldsb + kb] : sB[(int64_t)kb * ldsb + J];
            }
#pragma unroll
            for (int a = 0; a < WM; ++a)
#pragma unroll
                for (int b = 0; b < WN; ++b) {
                    const v16i p = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[b], af[a], zero, 0, 0, 0);
                    const float sigma = sa[a] * sb[b];
#pragma unroll
                    for (int r = 0; r < 16; ++r) acc[a][b][r] = __builtin_fmaf(sigma, (float)p[r], acc[a][b][r]);
                }
        }
        if (more) {
            ta.store(lds_a[buf ^ 1], tid);
            tb.store(lds_b[buf ^ 1], tid);
        }
        __syncthreads();
    }

    // Epilogue.  Lane owns row 32I + (lane & 31); accumulator r is column
    // 8(r/4) + 4(lane/32) + r%4 of block J.
    const int hc = 4 * (lane >> 5);
#pragma unroll
    for (int a = 0; a < WM; ++a)
#pragma unroll
        for (int b = 0; b < WN; ++b) {
            const int I = I0 + a, J = J0 + b;
            if (I >= nbM || J >= nbN) continue;
            const int64_t row = (int64_t)I * kBlock + frag_row;
            const int64_t col = (int64_t)J * kBlock + hc;
            if constexpr (OUT_I8) {
                float m = 0.0f;
#pragma unroll
                for (int r = 0; r < 16; ++r) m = fmaxf(m, fabsf(acc[a][b][r]));
                m = wave_max(m);
                const float sc = block_scale(m);
                int8_t *C = reinterpret_cast<int8_t *>(Cv);
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    uint32_t w = 0;
                    if (sc != 0.0f)
                        w = pack4(quant_code(acc[a][b][4 * g + 0], sc), quant_code(acc[a][b][4 * g + 1], sc),
                                  quant_code(acc[a][b][4 * g + 2], sc), quant_code(acc[a][b][4 * g + 3], sc));
                    *reinterpret_cast<uint32_t *>(C + row * ldc + col + 8 * g) = w;
                }
                if (lane == 0) sC[(int64_t)I * nbN + J] = sc;
            } else {
                float *C = reinterpret_cast<float *>(Cv);
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    *reinterpret_cast<float4 *>(C + row * ldc + col + 8 * g) =
                        make_float4(acc[a][b][4 * g + 0], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2],
                                    acc[a][b][4 * g + 3]);
            }
        }
}

template <int WM, int WN, int KB, bool A_KC, bool B_KC, bool OUT_I8>
hipError_t launch_cfg(int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda, const float *sA,
                      const int8_t *B, int64_t ldb, const float *sB, void *C, int64_t ldc, float *sC,
                      hipStream_t stream) {
    constexpr int BM = 2 * WM * kBlock, BN = 2 * WN * kBlock;
    const int64_t tilesM = (M + BM - 1) / BM, tilesN = (N + BN - 1) / BN;
    const int64_t ldsa = A_KC ? K / kBlock : M / kBlock;
    const int64_t ldsb = B_KC ? K / kBlock : N / kBlock;
    hipLaunchKernelGGL((k_gemm_i8bs<WM, WN, KB, A_KC, B_KC, OUT_I8>), dim3((unsigned)(tilesM * tilesN)),
                       dim3(kThreads), 0, stream, A, lda, sA, ldsa, B, ldb, sB, ldsb, (int)M, (int)N, (int)K, C,
                       ldc, sC, (int)tilesN);
    return hipGetLastError();
}

template <bool A_KC, bool B_KC>
hipError_t dispatch_out(bool out_i8, int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                        const float *sA, const int8_t *B, int64_t ldb, const float *sB, void *C, int64_t ldc,
                        float *sC, hipStream_t stream) {
    if (out_i8) return launch_cfg<2, 2, 2, A_KC, B_KC, true>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    return launch_cfg<2, 2, 2, A_KC, B_KC, false>(M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
}

}  // namespace

hipError_t launch_gemm(int transA, int transB, int64_t M, int64_t N, int64_t K, const int8_t *A, int64_t lda,
                       const float *sA, const int8_t *B, int64_t ldb, const float *sB, bool out_i8, void *C,
                       int64_t ldc, float *sC, hipStream_t stream) {
    if (M == 0 || N == 0) return hipSuccess;
    // A is k-contiguous when stored M x K (transA = 0); B when stored N x K (transB = 1).
    const bool akc = transA == 0, bkc = transB == 1;
    if (akc && bkc) return dispatch_out<true, true>(out_i8, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    if (akc && !bkc) return dispatch_out<true, false>(out_i8, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    if (!akc && bkc) return dispatch_out<false, true>(out_i8, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
    return dispatch_out<false, false>(out_i8, M, N, K, A, lda, sA, B, ldb, sB, C, ldc, sC, stream);
}

}  // namespace jf
