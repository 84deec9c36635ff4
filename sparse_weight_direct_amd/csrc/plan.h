// Internal types shared by the packer, the C ABI and the gfx950 kernels.
//
// Data layout used by the kernels (all sizes in 4-byte words):
//
//  * The padded input of one image is split into stride x stride phase planes: padded
//    position (yp, xp) lands in phase (yp % st, xp % st) at phase coordinates
//    (yp / st, xp / st).  A phase plane has HYp = ceil((H+2p)/st) rows of Pp = ceil((W+2p)/st)
//    words.  For stride 1 this is just the zero-padded image.
//  * Output (e, f) of image n reads, for tap (r, s), phase (r % st, s % st) at
//    (e + r/st, f + s/st): with stride folded into the phases every tap is a unit-stride
//    shift, so a run of consecutive "extended" output indices I = n*HYp*Pp + e*Pp + f maps
//    to consecutive LDS words for every tap.  Positions with e >= E or f >= F are junk
//    (computed, never stored).
//  * A workgroup owns 64*K consecutive extended indices (K per lane, 64 apart) and stages
//    the phase rows they touch, NRmax rows per phase, for Cc channels at a time:
//        LDS word = c_l*CHS + (py*st + px)*PH + row*Pp + col,  PH = NRmax*Pp, CHS = st*st*PH.
//  * Each stored non-zero (c, r, s, v) is re-encoded at pack time as
//        enc = (c % Cc)*CHS + ((r % st)*st + (s % st))*PH + (r / st)*Pp + (s / st)
//    so the inner loop is: one address add, K LDS reads 64 words apart, K FMAs.
#pragma once
#include <cstdint>
#include <vector>

namespace sc {

constexpr int kWaves = 8;               // wavefronts per workgroup (512 threads)
constexpr int kThreads = kWaves * 64;
constexpr int kLdsBudget = 64 * 1024;   // bytes of LDS per workgroup (2 per CU)

struct Geom {
  int M, C, R, S, H, W, st, pad;
  int E, F;        // output extent
  int Pp, HYp;     // phase plane row pitch and rows per image
  int Rr;          // distinct r / st values = (R-1)/st + 1
};

struct Plan {
  int K;           // extended output positions per lane (64 apart)
  int OCW;         // output-channel slots per wavefront
  int G;           // output-channel groups (workgroups per tile)
  int Cc;          // channels staged per chunk
  int nch;         // number of chunks = ceil(C / Cc)
  int NRmax;       // phase rows staged per phase plane
  int PH;          // words per phase plane = NRmax * Pp
  int CHS;         // words per staged channel = st*st*PH
  int lds_floats;  // staged words incl. tail slack for junk positions
  int lds_bytes;   // lds_floats*4 + row table
};

// Kernel arguments (by value).
struct KArgs {
  const float* x;
  float* y;
  const uint32_t* ent;    // sparse: pairs {enc, value bits}
  const int32_t* seg;     // sparse: pairs [slot][chunk] -> [beg, end) into ent
  const int* slot_row;    // sparse: [slot] -> output channel or -1
  const float* wd;        // dense baseline: M*C*R*S weights
  int N, C, H, W, M, E, F, R, S, st, pad;
  int Pp, HYp, img_ext;   // img_ext = HYp * Pp
  int NRmax, PH, CHS, Cc, nch, G;
  int lds_floats;
  long long ext_total;    // N * img_ext
};

bool make_geom(int M, int C, int R, int S, int H, int W, int st, int pad, Geom* g);
Plan choose_plan(const Geom& g, const std::vector<int32_t>& row_nnz);
int plan_nrmax(const Geom& g, int K);

// Launchers (kernels.hip).  Return a hipError_t value as int.
int launch_sparse(const Plan& p, const KArgs& a, void* stream, int nblocks);
int launch_dense(const Plan& p, const KArgs& a, void* stream, int nblocks);

}  // namespace sc
