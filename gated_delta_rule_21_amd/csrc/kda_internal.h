// kda_internal.h -- launch descriptors shared by the host entry points and
// the kernel translation units.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace kda {

struct DecodeArgs {
    bool f32io;
    const void *q, *k, *v;
    const float *z, *A, *beta;
    float *S;
    void *o;
    int N, H, dk, dv;
    hipStream_t stream;
};

// The fused decode step (bf16, dk = dv = d): features of the new token from
// xq, xk, xv and the carried window, the update of S, y = Sigmoid(g) *
// RMSNorm(o).
struct DecodeFusedArgs {
    const void *xq, *xk, *xv;
    const float *wq, *wk, *wv;
    const void *win_in;
    void *win_out;
    const float *z, *A, *beta;
    float *S;
    const void *gate;
    const float *norm_w;
    float eps;
    void *y;
    int N, H, d;
    hipStream_t stream;
};
int launch_decode_fused(const DecodeFusedArgs &a);

// Multi-token decode with replay: the replay window (inputs cached from the
// previous call, n_accept[n] of its Lr tokens committed now) and the new
// window of L tokens.  Inputs [N][len][H][d].
struct DecodeWindowArgs {
    bool f32io;
    const void *rk, *rv;
    const float *rz, *rbeta;
    const int32_t *n_accept;
    int Lr;
    const void *q, *k, *v;
    const float *z, *beta;
    int L;
    const float *A;
    float *S;
    void *o;
    int N, H, dk, dv;
    bool commit_window;
    hipStream_t stream;
};

// Feature path: q, k = L2Norm(Swish(ShortConv(x))), v = Swish(ShortConv(x)).
// x [T][H][d] io dtype, w [H][d][4] fp32, windows [N][3][H][3d] io dtype.
struct FeatureArgs {
    bool f32io;
    const void *xq, *xk, *xv;
    const float *wq, *wk, *wv;
    const int32_t *cu;
    int N, T, H, d;
    const void *win_in;
    void *win_out;
    void *q, *k, *v;
    hipStream_t stream;
    // chunk run of the pipelined fused prefill: only the tokens of chunks
    // [c_lo, c_hi) of the chunk table are written (nchunks: device count of
    // chunks), and the window is left to the caller
    const int4 *table = nullptr;
    const int32_t *nchunks = nullptr;
    int c_lo = 0, c_hi = 0;
};

// Output gate: y = Sigmoid(g) * RMSNorm(o), rows of dv.
struct GateArgs {
    bool f32io;
    const void *o, *g;
    const float *w;
    float eps;
    int T, H, dv;
    void *y;
    hipStream_t stream;
};

// Longest replay and window the decode-window kernel stages in LDS.
constexpr int kMaxWindow = 16;

// Workspace plan of the chunkwise prefill.  Offsets are bytes from the
// workspace base; every region is 256-byte aligned.
struct PrefillPlan {
    int max_chunks;          // ceil(T / 64) + N: an upper bound on the chunk count
    int P;                   // segment slots per sequence (1: no split)
    size_t slab_bytes;       // per (chunk, head) intermediate slab
    size_t off_meta;         // int32 [N + 1] per-sequence first chunk, then [1] total
    size_t off_table;        // int32x4 [max_chunks]: sequence, first token, length, -
    size_t off_null;         // the null row: z = -inf [dk] fp32, zeros [max(dk,dv)] io dtype, beta = 0
    size_t off_ckoff;        // int32 [N + 1]: first checkpoint of every sequence, then the total
    size_t off_segs;         // int32x4 [N * P]: sequence, first chunk, end chunk, flags
    size_t off_trans;        // P > 1: fp32 [N * P][H][2][dk * dk]: M row-major, then S~ in state layout
    size_t off_sin;          // P > 1: fp32 [N * P][H][dv][dk] incoming state of every segment
    size_t off_slabs;        // slabs, head-major: [H][max_chunks]
    int blocks;              // block pipeline: chunk blocks (1: off)
    size_t off_claims;       // blocks > 1: int32 [blocks] item counters
    size_t off_carry;        // blocks > 1: fp32 [N][H][dv][dk] state between blocks
    bool staged;             // pipelined fused call: q, k, v staged by the feature kernel
    size_t off_qkv;          // staged: io dtype [3][T][H][dk] q, k, v
    size_t total;
};

// Largest segment count per sequence (at most 64: the combine kernel reads
// a sequence's segment records one per lane of a wave).
constexpr int kMaxSegments = 16;
static_assert(kMaxSegments <= 64, "segment records per wave");

// The fused prefill's extra inputs and outputs (bf16 path): the feature
// path in front of the recurrence and the output gate behind it.
struct FusedIO {
    const void *xq, *xk, *xv;    // [T][H][d] projected inputs, io dtype (q, k, v are computed from them)
    const float *wq, *wk, *wv;   // [H][d][4] ShortConv taps
    const void *win_in;          // [N][3][H][3d] carried conv window, or NULL (zeros)
    void *win_out;               // the window after the call, or NULL; may be win_in
    const void *g;               // [T][H][dv] gate projection, io dtype
    const float *w;              // [dv] RMSNorm weight
    float eps;
};

struct PrefillArgs {
    bool f32io;
    const void *q, *k, *v;
    const float *z, *A, *beta, *h0;
    const int32_t *cu;
    int N, T, H, dk, dv;
    void *o;
    float *hT;
    float *ck;               // checkpoints [T / ck_interval][H][dv][dk] fp32, or NULL
    int32_t *ck_offsets;     // caller's copy of the per-sequence checkpoint offsets, or NULL
    int ck_interval;         // tokens between checkpoints, a multiple of 64
    unsigned char *ws;
    PrefillPlan plan;
    hipStream_t stream;
    // fused call: q, k, v are NULL and o receives y = Sigmoid(g) * RMSNorm(o)
    const FusedIO *fused = nullptr;
};

// Workspace plan of the prefill backward: the forward's own workspace, its
// discarded outputs, the state at every chunk boundary, and one fp32 record
// per (chunk, head).
struct BackwardPlan {
    PrefillPlan fwd;         // at off_fwd
    int ck_cap;              // T / 64: chunk-boundary states stored
    size_t off_fwd, off_o, off_ck, off_items, off_dA, total;
};

struct BackwardArgs {
    bool f32io;
    const void *q, *k, *v;
    const float *z, *A, *beta, *h0;
    const int32_t *cu;
    int N, T, H, d;
    const void *dO;          // [T][H][d] io dtype
    const float *dhT;        // [N][H][d][d] or NULL
    float *gq, *gk, *gv, *gz, *gbeta, *gA, *gh0;   // fp32 gradients; gh0 may be NULL
    unsigned char *ws;
    BackwardPlan plan;
    hipStream_t stream;
};

// `fused`: the plan of the fused call, which stages q, k, v in the workspace
// when it is pipelined.
bool plan_prefill(int N, int T, int H, int dk, int dv, bool f32io, int P, int blocks, PrefillPlan *plan,
                  bool fused = false);
// Chunk blocks of the pipelined prefill for these sizes when the caller asks
// for the automatic choice (1: not pipelined).
int choose_blocks(int N, int T, int H, int d, bool fused = false);
bool plan_backward(int N, int T, int H, int d, bool f32io, int P, BackwardPlan *plan);
// Segment count the prefill uses for these sizes when the caller asks for
// the automatic choice.
int choose_segments(int N, int T, int H, int d);
size_t slab_bytes(int dk, int dv, bool f32io);

int launch_decode(const DecodeArgs &a);
int launch_decode_window(const DecodeWindowArgs &a);
int launch_features(const FeatureArgs &a);
// Only the carried conv window of the feature path (win_out from x and win_in).
int launch_conv_window(bool f32io, const void *xq, const void *xk, const void *xv, const int32_t *cu, int N, int T,
                       int H, int d, const void *win_in, void *win_out, hipStream_t stream);
int launch_output_gate(const GateArgs &a);
int launch_prefill(const PrefillArgs &a);
int launch_prefill_backward(const BackwardArgs &a);
// Intra-chunk kernels (kda_intra.hip: bf16 path; kda_intra_f32.hip: fp32
// path), D = 32, 64, 128.
template <int D>
int launch_intra_bf16(const PrefillArgs &a, const int32_t *meta, const int4 *table, const float *null_row,
                      unsigned char *slabs, int item_lo = 0, int item_hi = 0, int *claims = nullptr);
template <int D>
int launch_intra_f32(const PrefillArgs &a, const int32_t *meta, const int4 *table, unsigned char *slabs);

}  // namespace kda
