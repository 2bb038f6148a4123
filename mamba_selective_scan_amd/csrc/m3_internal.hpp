// m3_internal.hpp -- parameter blocks and launcher declarations shared by the
// host dispatch (m3_api.cpp) and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace m3 {

// Rows of one matrix-core block: (token, rank) pairs, rank fastest.
constexpr int kBlockRows = 64;

// Option bits of ScanParams::flags / StepParams::flags (the values of the public M3_FLAG_*).
constexpr uint32_t kFlagNorm = 1u << 0, kFlagPartialRope = 1u << 1, kFlagAPerToken = 1u << 2,
                   kFlagDtSoftplus = 1u << 3, kFlagLamSigmoid = 1u << 4, kFlagHalfSplit = 1u << 5;

struct ScanParams {
    // sizes
    int64_t B, T;
    int H, P, N, R;
    int TB;    // tokens per block (TB * R <= kBlockRows)
    int nblk;  // blocks per (batch, head) sequence
    int nseg;  // output segments per sequence (a workgroup walks one segment's blocks in order)
    int bps;   // blocks per output segment
    int nsub;  // state sub-segments per sequence, covering the blocks of segments 0 .. nseg-2
    int sbps;  // blocks per state sub-segment (divides bps)
    int ncg;   // column groups: P is split across workgroups in groups of at most 64 columns
    uint32_t flags;
    float eps;
    int nr;  // rotated pairs (N/2 unless the rotation is partial): theta and angle hold nr per token / sequence
    // inputs
    const void *x, *Bm, *Cm;
    const float *dt, *lam, *theta, *A, *D;  // A: [H], or [B, T, H] with kFlagAPerToken
    const float *bnw, *cnw, *bbias, *cbias;
    const float *dtbias;  // [H] or NULL (read with kFlagDtSoftplus)
    const void *z;        // gate input laid out like y (rank-free with mz), or NULL
    const float *mx, *mz, *mo;  // MIMO projection vectors [H, R, P], or NULL
    // row strides (elements between tokens b*T + t), never 0: x, B, C, dt, lambda, theta,
    // A (per token), z, y
    int64_t rsx, rsb, rsc, rsdt, rslam, rsth, rsa, rsz, rsy;
    void *y;
    // carried state
    const float *h0, *pB0, *px0, *ang0;  // initial (NULL = zeros)
    float *h1, *pB1, *px1, *ang1;        // final (NULL = not requested)
    // workspace
    int np2;      // pairs padded to the tile height (NP / 2): pitch of pseg and cseg
    int pp;       // columns per workgroup, padded (PP)
    // per state sub-segment, written by the state kernel:
    float *Sagg;  // [B*H*ncg][nsub][NP*PP] state contributed by the sub-segment, from zero, in
                  //   its end frame, stored in matrix-core fragment order (tile, lane, slot)
    float *lseg;  // [B*H][nsub]         sum of dt*A over the sub-segment
    float *pseg;  // [B*H][nsub][np2]    sub-segment angle total reduced to [0, 2 pi); padded pairs 0
    float *cseg;  // [B*H][nsub][np2][2] (cos, sin) of that angle; padded pairs (1, 0)
    // per output segment, written by the prefix kernel (NULL when it does not run):
    float *Hin;   // [B*H*ncg][nseg][NP*PP] incoming state in the frame of the segment's first
                  //   block, fragment order
    unsigned int *dbg;  // debug builds: [count of failed device checks, largest failing line]
};

struct StepParams {
    int64_t B;
    int H, P, N, R;
    uint32_t flags;
    float eps;
    int nr;  // rotated pairs
    const void *x, *Bm, *Cm;
    const float *dt, *lam, *theta, *A, *D;  // A: [H], or [B, H] (one token) with kFlagAPerToken
    const float *bnw, *cnw, *bbias, *cbias;
    const float *dtbias;
    const void *z;
    const float *mx, *mz, *mo;  // MIMO projection vectors [H, R, P], or NULL
    int64_t rsx, rsb, rsc, rsdt, rslam, rsth, rsa, rsz, rsy;  // row strides (one token: row = b)
    void *y;
    float *h, *pB, *px, *ang;
    unsigned int *dbg;  // debug builds: failed device checks (as ScanParams::dbg)
};

// Gradients of a scan (reverse-mode), chunk by chunk: 64 (token, rank) rows per chunk,
// states before and adjoints after every chunk in the workspace.
struct BwdParams {
    int64_t B, T;
    int H, P, N, R;
    uint32_t flags;
    float eps;
    int nr;
    int hs;  // pairs (i, i + N/2) (the half-split pairing, N 64 or 128) instead of (2i, 2i + 1)
    // forward inputs (as for ScanParams)
    const void *x, *Bm, *Cm;
    const float *dt, *lam, *theta, *A, *D;
    const float *bnw, *cnw, *bbias, *cbias, *dtbias;
    const void *z;
    const float *h0, *pB0, *px0, *ang0;      // initial state or NULL
    // upstream gradients
    const void *dy;                           // like y
    const float *dh1, *dpB1, *dpx1, *dang1;  // of the final state, or NULL
    // per-element gradients
    void *dx, *dB, *dC, *dz;                  // io dtype
    float *ddt, *dlam, *dtheta, *dAt;         // dAt: per-token A gradient (kFlagAPerToken) or NULL
    float *dh0, *dpB0, *dpx0, *dang0;         // or NULL
    // parameter gradients (each may be NULL); summed by bwd_reduce_kernel
    float *dA, *dD, *dbnw, *dcnw, *dbb, *dcb, *ddtb;
    // plan
    int nck;   // chunks per sequence (64 / R tokens each)
    int vec;   // 16-byte staging loads (P R, N R multiples of 16 / element size, nr of 4)
    int pw;    // floats per partial-sum record (one per (sequence, chunk))
    // workspace (fp32)
    float *Sst;    // [BH][nck][N][P] chunk state sums -> (in place) state before each chunk
    float *Ust;    // [BH][nck][N][P] chunk adjoint sums -> (in place) adjoint after each chunk
    float *lsum;   // [BH][nck]       sum of log alpha over the chunk
    float *phic;   // [BH][nck][N/2]  sum of theta over the chunk
    float *thst;   // [BH][N/2]       angle before the last chunk
    float *G0w;    // [BH][N][P]      adjoint of the initial state (global frame)
    float *hfin;   // [BH][N][P]      state after the last chunk (that chunk's frame)
    float *tot;    // [BH][nck][N/2]  angle gradient sum of the chunk -> (in place) of the later chunks
    float *dsc;    // [BH][T][3]      d log alpha, d gamma, d eta per token
    float *deta0;  // [BH]            d eta of the initial state
    float *part;   // [BH][nck][pw]   parameter partial sums
    unsigned int *dbg;  // debug builds: failed device checks (as ScanParams::dbg)
};
hipError_t launch_bwd(bool bf16, const BwdParams &p, hipStream_t stream);

// N-axis permutation between the half-split pairing (component c of pair i at i + c N/2) and
// the kernels' adjacent pairing (at 2 i + c), of a tensor viewed as [outer][N][inner] with
// elements of esize bytes (2 or 4); to_kernel: half-split -> adjacent, else the inverse.
hipError_t launch_perm_n(const void *in, void *out, int64_t outer, int N, int inner, int esize, bool to_kernel,
                         hipStream_t stream);

// Tile variant chosen by the host.
enum TileMode { kTileGen = 0, kTileVec = 1, kTileMimo = 2 };
struct TileShape {
    int np;    // N padded: 32, 64 or 128
    int pp;    // columns per workgroup, padded: 32 or 64
    int mode;  // kTileVec: rank 1 with N % 8 == 0 and P % 8 == 0 (16-byte accesses);
               // kTileMimo: bf16, rank 2, 4 or 8, N % 8 == 0, P % 8 == 0 (16-byte accesses);
               // kTileGen: anything else (element accesses)
    bool pj = false;  // the call has MIMO projections: the kernels that read them (not kTileVec)
    bool hs = false;  // half-split pairing in the kernels (kTileVec with N = np >= 64, no prefix pass)
};

hipError_t launch_seg_state(bool bf16, const TileShape &ts, const ScanParams &p, hipStream_t stream);
hipError_t launch_seg_prefix(const TileShape &ts, const ScanParams &p, hipStream_t stream);
hipError_t launch_seg_output(bool bf16, const TileShape &ts, const ScanParams &p, hipStream_t stream);
size_t seg_kernel_lds_bytes(bool output, bool bf16, const TileShape &ts);
hipError_t launch_fill_state(const ScanParams &p, hipStream_t stream);
hipError_t launch_step(bool bf16, const StepParams &p, hipStream_t stream);

}  // namespace m3
