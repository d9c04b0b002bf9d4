"""Plain CPU oracle of the FS-L forward. Test infrastructure only: the product
path (the HIP library and its binding) never imports this package."""
