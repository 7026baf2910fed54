// Workgroup id -> (query head, dim part) of the merge launch (merge.hip).
//
// The launch has batch * Hq * parts workgroups, parts = D / (dims per
// workgroup).  Ids run group-major: id mod groups is the KV group (groups =
// batch * hkv, hkv counting a split KV head's chunks), then the dim part,
// then the head within the group.  The step launch runs a group's
// workgroups slice-major, ids congruent mod groups, and the hardware deals
// ids round-robin to the 8 XCDs: with a multiple of 8 groups, a group's
// merge workgroups then land on the XCD its step workgroups ran on.
#pragma once

#include <hip/hip_runtime.h>

namespace mac {

struct MergeCoords {
  int grp;   // KV group: b * hkv + kvh
  int b;     // sequence
  int h;     // query head within the sequence
  int hi;    // query head within the group
  int q;     // dim part
};

__host__ __device__ __forceinline__ MergeCoords merge_coords(int id, int batch, int hkv, int group,
                                                             int parts) {
  const int groups = batch * hkv;
  MergeCoords m;
  m.grp = id % groups;
  const int rest = id / groups;
  m.q = rest % parts;
  m.hi = rest / parts;
  m.b = m.grp / hkv;
  m.h = (m.grp % hkv) * group + m.hi;
  return m;
}

}  // namespace mac
