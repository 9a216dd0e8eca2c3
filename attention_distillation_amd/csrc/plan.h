// Host-side planning: split factors, workspace layout and argument checks.
#pragma once
#include <string>
#include <vector>

#include "../../include/kvsculpt.h"
#include "kvs_internal.h"

namespace kvs {

struct Region {
  size_t off = 0, bytes = 0;
};

struct Plan {
  int P = 0, d = 0, Z = 0, n = 0, npad = 0, kmax = 0, kpadmax = 0, H = 10;
  long long ktot = 0, kpadtot = 0, mtot = 0, stot = 0;
  long long gtot = 0;          // 128x128 Gram tiles of all problems
  long long gtot4 = 0;         // 256x256 Gram tiles of all problems
  int Cref = 1, C = 1, Cn = 1, Cg = 1, Cq = 1, Crf = 1, nblk = 1, nchv = 1, nchd = 1;
  std::vector<ProbInfo> info;
  std::vector<int> chol_wgs;   // workgroups of Cholesky launch j = -1 .. kpadmax/64 - 1 (index j + 1)
  int chol_S = 1;              // panels per trailing pass of the Cholesky
  // workspace regions
  Region r_info, r_state, r_status, r_yref, r_lseref, r_St, r_Opart, r_Mpart, r_Lpart, r_G, r_e,
      r_crow, r_part, r_dK, r_grad, r_Mg, r_M, r_tr, r_mu, r_cinfo, r_X, r_imp, r_hpart, r_g, r_p, r_Kt,
      r_S, r_Yh, r_idx, r_flags, r_loss, r_Kc, r_Vc, r_cnt, r_Dinv, r_R, r_coff, r_K8, r_Kscl;
  size_t ws_bytes = 0;
  // persistent L-BFGS state buffer (kvs_lbfgs_* calls)
  Region s_state, s_g, s_p, s_S, s_Yh;
  size_t state_bytes = 0;
};

// Fills plan from the batch; returns an error text or empty.
std::string make_plan(const kvs_batch* b, const kvs_opts* o, Plan* plan);

// Key chunks of the split forward for `keys` keys: at most `cap`, enough
// workgroups for the part, and no chunk left empty by rounding the chunk
// length up to whole 64-key tiles.
int key_chunks(int P, int n, int keys, int cap);

// Workspace of the use-side evaluation: split-key partials of the three
// caches (compress zone, retain zone, compressed pairs) in adjacent planes,
// the two merged outputs and the error partials.
struct UsePlan {
  int P = 0, d = 0, Z = 0, n = 0, m = 0, kmax = 0;
  long long ktot = 0;
  int Cz = 0, Cr = 0, Cc = 0, nblk = 0;
  std::vector<ProbInfo> info;
  Region r_info, r_Opart, r_Mpart, r_Lpart, r_Of, r_Oc, r_lf, r_lc, r_part;
  size_t ws_bytes = 0;
};
std::string make_use_plan(const kvs_batch* b, int m, UsePlan* plan);

template <typename T>
inline T* at(void* base, const Region& r) {
  return reinterpret_cast<T*>(static_cast<char*>(base) + r.off);
}

}  // namespace kvs
