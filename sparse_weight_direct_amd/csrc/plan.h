// Internal types shared by the packer, the C ABI and the gfx950 kernels.
//
// Data layout used by the kernels (all sizes in 4-byte words):
//
//  * The padded input of one image is split into stride x stride phase planes: padded
//    position (yp, xp) lands in phase (yp % st, xp % st) at phase coordinates
//    (yp / st, xp / st).  A phase plane has HYp = ceil((H+2p)/st) rows of Pp = ceil((W+2p)/st)
//    words.  For stride 1 this is just the zero-padded image.
//  * Wide layout (stride 1, W % 4 == 0, pad <= 2, pad < S): input column x sits at phase column x + 4
//    and Pp = W + 4, so every aligned group of 4 words is 4 input words or 4 zeros and can be
//    copied with 16-byte loads; output column f then sits at extended column f + 4 - pad.
//    In general input column x sits at phase column (x + xoff) / st (xoff = pad, or 4 in the
//    wide layout) and output column f at extended column f + cshift (cshift = xoff - pad).
//  * Output (e, f) of image n reads, for tap (r, s), phase (r % st, s % st) at
//    (e + r/st, f + s/st): with stride folded into the phases every tap is a unit-stride
//    shift, so a run of consecutive "extended" output indices I = n*HYp*Pp + e*Pp + f maps
//    to consecutive LDS words for every tap.  Positions with e >= E or f >= F are junk
//    (computed, never stored).
//  * A workgroup owns a tile of 64*K consecutive extended indices [I0, I0 + 64K) (K per
//    lane, 64 apart; quad plans below: 504).  For every phase plane it stages exactly the range the tile's taps
//    read, PL = 64K + (Rr-1)*Pp + (S-1)/st consecutive phase-plane words starting at I0
//    (rows of the next image and padding included as zeros; for stride > 1 PL is rounded up
//    to a multiple of 64, so every 64-word block lies in one phase plane), for Cc channels
//    at a time:
//        LDS word = c_l*CHS + (py*st + px)*PL + (J - I0)   for phase-plane index J,
//    with the channel stride CHS = st*st*PL rounded up to a multiple of 64 words, so that
//    every channel is nblk = CHS/64 blocks of 64 words and a block's source offsets are
//    the same for every channel (they differ by a multiple of H*W).
//  * Each stored non-zero (c, r, s, v) is re-encoded at pack time as
//        enc = (c % Cc)*CHS + ((r % st)*st + (s % st))*PL + (r / st)*Pp + (s / st)
//    so lane l, position b reads LDS word enc + l + 64*b: one address add, K LDS reads 64
//    words apart and K FMAs per non-zero.  enc < slot_words < 2^16, so it also fits the
//    16-bit field of the 4-byte entry form.
//  * Quad plans (Plan::quad): lane l holds the 4 consecutive positions 4l..4l+3 of two
//    blocks 252 apart, so a tile is 504 positions (lane 63 computes junk that is never
//    stored: its words only feed lane 62 through a one-lane shift).  A non-zero's words for
//    the lane are then the aligned quad at word 4l + (enc & ~3) shifted by enc & 3 (the
//    tap's class): two 16-byte LDS reads per non-zero, the shifted words taken from the next
//    lane's quad by a DPP FMA.  Each slot's non-zeros of a chunk are sorted by class, the
//    header gives the four class counts, and an entry holds the byte offset of its aligned
//    quad.  PL = 508 + (Rr-1)*Pp + (S-1)/st covers lane 63's reads.
#pragma once
#include <cstdint>
#include <vector>

namespace sc {

constexpr int kLdsMax = 160 * 1024;     // LDS per CU
constexpr int kMaxDepth = 4;            // most LDS ring slots (ready/done counter pairs)

struct Geom {
  int M, C, R, S, H, W, st, pad;
  int E, F;        // output extent
  int Pp, HYp;     // phase plane row pitch and rows per image
  int Rr;          // distinct r / st values = (R-1)/st + 1
  int wide;        // 1: wide layout (16-byte staging loads possible)
  int xoff;        // padded-column offset of input column 0 (pad, or 4 in the wide layout)
  int cshift;      // extended column of output column 0 (xoff - pad)
};

struct Plan {
  int K;           // extended output positions per lane (64 apart)
  int OCW;         // output-channel slots per wavefront
  int NW;          // wavefronts per workgroup: NW-1 consumers (OCW slots each) + 1 producer
  int G;           // output-channel groups (work units per tile)
  int Cc;          // channels staged per chunk
  int nch;         // number of chunks = ceil(C / Cc)
  int PL;          // staged words per phase plane >= 64K + (Rr-1)*Pp + (S-1)/st (a multiple
                   // of 64 for stride > 1)
  int CHS;         // words per staged channel = st*st*PL rounded up to a multiple of 64
  int nblk;        // 64-word blocks per staged channel = CHS / 64 (CHS a multiple of 256
                   // in the wide layout: nblk/4 blocks of 256 words)
  int D;           // LDS ring slots: D-1 chunks in flight
  int slot_words;  // words of one ring slot (the chunk's input rows) = Cc*CHS
  int lds_bytes;   // D ring slots + ready/done counters + block-start table
  int span_images; // most images one tile's staged range can touch
  int step_permille;  // 1000 * sum over chunks of the busiest wavefront's entries / mean
  int nbuf;        // LDS partial-sum buffers per workgroup (pieces of split rows)
  int h16;         // entry format: 0 {LDS offset, fp32 weight} (8 bytes), 1 fp16 weight in
                   // bits 15..0 and the LDS offset in bits 31..16 (4 bytes)
  int quad;        // 1: quad plan (K = 8: two blocks of 4 consecutive positions per lane)
  int tp;          // extended positions per tile: 64*K, or kQuadTile for quad plans
  int ring_words;  // quad plans: LDS word offset of the consumers' entry rings (a multiple
                   // of 4; each consumer has 128 entries of 8 bytes there)
};

constexpr int kQuadTile = 504;        // 63 lanes x 4 positions x 2 blocks
constexpr int kQuadBlock = 252;       // words between a lane's two quads
constexpr int kQuadRingBytes = 1024;  // per consumer: two groups of 64 entries

// Row schedule.  A row longer than a consumer's fair share of a group's non-zeros is split
// into pieces held by different consumers of its group: in every chunk, piece p of P takes
// a contiguous part of the row's entries of that chunk (piece_range).  Piece 0's slot
// owns the row: after the unit's last chunk it adds the other pieces' partial sums, which
// they leave in LDS buffers, in piece order, and stores.
struct Sched {
  std::vector<int32_t> slot_row;   // kernel table per (group, consumer, slot): >= 0 output
                                   // channel (whole row or piece 0), -1 empty, <= -2: a
                                   // later piece writing partial buffer -2 - value
  std::vector<int32_t> slot_comb;  // kernel table: for piece 0 of a split row,
                                   // (first partial buffer << 8) | (pieces - 1); else 0
  std::vector<int32_t> src_row;    // row whose piece a slot holds, -1 empty
  std::vector<int32_t> piece;      // piece index of the slot
  std::vector<int32_t> npieces;    // pieces of that row
  int nbuf = 0;                    // partial buffers of all groups (each used by one group)
  int32_t max_wave_nnz = 0;        // largest non-zero count of one consumer
  int32_t split_pieces = 0;        // pieces beyond the first, over all rows
};

// Entries [pb, pe) of piece p of P of a chunk's entry range [b, e).
inline void piece_range(int b, int e, int p, int P, int* pb, int* pe) {
  *pb = b + (int)((long long)(e - b) * p / P);
  *pe = b + (int)((long long)(e - b) * (p + 1) / P);
}

// Kernel arguments (by value).
struct KArgs {
  const float* x;
  float* y;
  const uint32_t* ent;    // sparse: entries {enc, value bits}, or one word each (Plan::h16)
  const int32_t* seg;     // sparse: [(group*NC + consumer)*(nch+1) + k] -> first entry of block k
  const int* slot_row;    // sparse: [group][consumer][slot] -> Sched::slot_row
  const int* slot_comb;   // sparse: [group][consumer][slot] -> Sched::slot_comb
  int N, C, H, W, M, E, F, R, S, st, pad;
  int Pp, HYp, img_ext;   // img_ext = HYp * Pp
  int xoff, cshift;       // see Geom
  int wide16;             // 1: stage rows with 16-byte loads (wide layout, aligned input)
  int nsb;                // staging blocks per channel: nblk/4 of 256 words (wide16) or nblk
  int PL, CHS, nblk, Cc, nch, G, D, slot_words;
  int nbuf;               // partial-sum buffers (split rows)
  int HW;                 // H * W
  int ntiles;             // tiles of tp extended positions
  int tp;                 // extended positions per tile (Plan::tp)
  int ring_words;         // quad plans: LDS word offset of the entry rings (Plan::ring_words)
  long long x_words;      // N * C * H * W
  long long ext_total;    // N * img_ext
  uint32_t* status;       // the handle's device status word (bit 0: a bounded wait gave up)
  int spin_limit;         // sleeps before a wait gives up
};

bool make_geom(int M, int C, int R, int S, int H, int W, int st, int pad, Geom* g);
// Launch plan for the CSR filter matrix (rowptr, col): also schedules rows onto wavefront
// slots (slot_row) and sizes each wavefront's per-chunk block of non-zeros.
// k_cap / ocw_cap > 0 cap K and OCW; d > 0 sets the ring depth (default 3).
// quad = 1 asks for a quad plan (K = 8, OCW of 3, 5 or 9).
Plan choose_plan(const Geom& g, const std::vector<int32_t>& rowptr, const std::vector<int32_t>& col,
                 Sched* sched, int k_cap = 0, int ocw_cap = 0, int d = 0, int quad = 0);
int plan_pl(const Geom& g, int K, int quad = 0);

// Header entries at the start of a wavefront's per-chunk block of non-zeros.
int block_header(int OCW);

// CUs of the current device and workgroups of the plan's kernel that fit on one CU; also
// raises the kernel's dynamic LDS limit to the plan's size (kernels.hip).  Returns a
// hipError_t.  The persistent grid is min(units, cus * per_cu) workgroups, each taking a
// contiguous run of units.
int occupancy(const Plan& p, int* cus, int* per_cu);

// Launchers (kernels.hip).  Return a hipError_t value as int.
int launch_sparse(const Plan& p, const KArgs& a, void* stream, int nblocks);

// Second mapping ("Escoin" dataflow, escoin.hip): a pad_in kernel writes the zero-padded
// input (planes of Hp x Wp words) to a workspace, then one workgroup per (output channel,
// tile of 256*kEscoinP output positions, image) keeps its CSR row in LDS and reads the
// padded input through the caches.  Entries are {(c*Hp + r)*Wp + s, fp32 value bits}.
constexpr int kEscoinP = 4;      // output positions per thread (256 apart)
constexpr int kEscoinChunk = 4096;  // most row entries held in LDS at once

struct EscoinArgs {
  int N, C, H, W, M, E, F, st, pad;
  int Hp, Wp;        // padded plane: H + 2 pad, W + 2 pad
  int img_words;     // C * Hp * Wp
  int tiles;         // ceil(E*F / (256 * kEscoinP))
  int chunk;         // row entries per LDS pass: min(longest row, kEscoinChunk), >= 1
};

int launch_escoin(const EscoinArgs& a, const float* x, float* xp, float* y, const uint32_t* ent,
                  const int32_t* rowptr, void* stream);

// The static workspace of escoin.hip (kScratchBytes, 256-byte aligned): *ptr receives its
// device address on the current device, resolved once per device (hipGetSymbolAddress) and
// cached.  Returns a hipError_t.
constexpr long long kScratchBytes = 32LL << 20;  // SC_NOALLOC_SCRATCH_BYTES
int scratch_address(void** ptr);

// Dense direct baseline (dense.hip): every tap of a dense M x C x R x S filter tensor on the
// device.  The caller fills the geometry; the launcher sets tgroups and groups.  Input and
// output must each be < 2^31 bytes (32-bit buffer offsets).
struct DenseArgs {
  int C, H, W, M, R, S, st, pad, E, F;
  int EF, MEF, CHW, HW4;   // E*F, M*E*F, C*H*W, H*W*4
  int RS, CRS;             // R*S, C*R*S
  int qtot;                // N*E*F output positions per channel (< 2^31)
  uint32_t x_bytes, y_bytes;
  int tgroups, groups;     // position-tile groups and output-channel groups
};
// Tile shape of a launch: K positions per lane, MG output channels per wavefront, picked for
// the layer and the device's SIMD count.
void dense_pick(const DenseArgs& a, int simds, int* K, int* MG);
int launch_dense(DenseArgs a, const float* w, const float* x, float* y, int simds, void* stream);

}  // namespace sc
