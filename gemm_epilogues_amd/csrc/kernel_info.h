// One row of the kernel resource table that build.py generates from the
// compiler's resource report of this library (host only; see fc_kernel_info).
#ifndef FC_KERNEL_INFO_H
#define FC_KERNEL_INFO_H

namespace fc {

struct KernelInfoRow {
    const char *name;       // demangled, without the parameter list
    int vgprs, agprs, sgprs, lds_bytes, scratch_bytes, waves_per_simd;
};

extern const KernelInfoRow kKernelInfo[];
extern const int kKernelInfoCount;

}  // namespace fc

#endif
