"""he_database_scan_amd -- the PIR server's database-multiplication scan on
AMD Instinct MI355X (gfx950): RowSel in the NTT/RNS domain and the scalar-HE
(Regev) INT8 x uint32 product mod 2^32, as the C-ABI library libpirscan with a
thin Python binding (:mod:`he_database_scan_amd.pirscan`)."""
from . import pirscan  # noqa: F401

__all__ = ["pirscan"]
